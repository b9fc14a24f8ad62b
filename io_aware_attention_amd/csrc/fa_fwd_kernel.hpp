// fa_fwd_kernel.hpp -- fused FlashAttention forward kernels for gfx950 (CDNA4).
//
// One workgroup owns one tile of BR = 32*WAVES query rows of one (batch, query
// head) and streams the key/value rows of the matching K/V head through LDS in
// blocks of BC rows.  Each 64-lane wavefront owns 32 query rows.  For every
// key/value block the wavefront
//
//   1. computes the transposed score tile S^T = K_blk Q_w^T (BC x 32) on the
//      matrix cores (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation);
//   2. masks keys past the causal diagonal or past N (only in blocks that need it);
//   3. updates the running row maximum m, row sum l and output accumulator O by
//      the online-softmax recurrence ("MCU 上 Transformer 模型的 Flash Attention
//      实现…", §二, flowchart: m_new = max(m_old, rowmax S), P = exp(S - m_new),
//      l_new = e^(m_old - m_new) l_old + rowsum P, O_new = e^(m_old - m_new) O_old + P V),
//      in base 2 with the scale and log2(e) folded into one multiplier.  The quotient
//      O/l and m + log2 l do not depend on which m is used as long as the weights
//      stay in range, so m is only moved when it must be: the block's weights are
//      first taken against the current m, and only if a lane's sum of them exceeds
//      a cap (so some weight might) is the block maximum taken, O and l rescaled,
//      and the weights recomputed;
//   4. accumulates O^T += V_blk^T P^T on the matrix cores, P rounded to the input
//      type; the row sum l adds those same rounded values.
//
// O is normalised once after the last block (§三 of the same page, final
// normalisation) and written with lse = ln 2 * (m + log2 l).  Nothing of size N x N
// is ever stored ("FlashAttention (VI)", sections on tiling and kernel fusion).
//
// Register layouts (32x32 MFMA): lane L holds operand row/column L % 32 and the
// eight consecutive k-slots 8*(L/32) .. 8*(L/32)+7; accumulator register r of lane L
// holds row 8*(r/4) + 4*(L/32) + r%4 of column L % 32.  With the score tile
// transposed, each lane owns one query row (its column), and a row's 2*16 scores sit
// in lanes L and L^32: row reductions are in-lane plus one v_permlane32_swap.  The
// same accumulator registers, converted to 16-bit, are directly the B operand of the
// P.V product; V stays row-major in LDS and its A operand (Vᵀ fragments) comes from
// transposing 8-byte LDS reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_args.hpp"

namespace fa355 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kTau = 8.0f;                 // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, 32-bit dwords (gfx9 family)

template <typename T> struct Mfma;
template <> struct Mfma<BF16> {
    // bf16 rounds P by up to 2^-8 relative, too coarse for a 1e-3 logsumexp: the
    // lse keeps its own fp32 sum of the unrounded P.
    static constexpr bool kSeparateLseSum = true;
    // ... and too coarse to normalise O by that sum: O is divided by the sum of the
    // rounded weights the P.V product used.
    static constexpr bool kRoundedRowSum = true;
    // Largest lane sum of weights accepted without a rescale: bounds every weight,
    // hence O's accumulator at N 2^16 max|V|.
    static constexpr float kSumCap = 65536.0f;
    static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    // Two fp32 values -> two bf16, round to nearest even (v_cvt_pk_bf16_f32).
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        f32x2_t v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    }
    // acc + lo + hi of a packed pair (v_dot2c_f32_bf16 against (1, 1)).
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), one, acc, false);
    }
};
template <> struct Mfma<F16> {
    static constexpr bool kSeparateLseSum = false;   // fp16 rounds P by <= 2^-11
    // Rounding moves the row sum by at most 2^-11 relative: the fp32 sum of the
    // unrounded weights normalises O as well (and spares the packed-pair dot
    // products, which wait for the matrix pipe while an MFMA runs).
    static constexpr bool kRoundedRowSum = false;
    // Weights are rounded to fp16 (largest finite 65504): a lane sum of rounded
    // weights at most 2^15 keeps each below that (an overflow to inf fails the test).
    static constexpr float kSumCap = 32768.0f;
    static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    // Two fp32 values -> two fp16, round to nearest even (v_cvt_f16_f32).
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        f32x2_t v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    }
    // acc + lo + hi of a packed pair (v_dot2c_f32_f16 against (1, 1)).
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pair), one, acc, false);
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kRsrcWord3);
}

// 16-byte load; offsets at or past the resource size read as zero.
__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// 16 bytes per lane from a buffer straight into LDS: lane L's data lands at
// lds + 16 L (lds is wave-uniform).  Out-of-range lanes write zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *lds, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)   // LDS pointers exist only in the device pass
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 0);
#else
    (void)r; (void)lds; (void)voff;
#endif
}

// Debug build (-DFA355_LDS_POISON=1): before each LDS stage is refilled, every byte
// of it is set to 0xff -- a NaN as bf16, fp16, fp32 and e4m3 -- and each refill is
// waited for before the block in the other stage is computed.  A read of LDS that
// no copy wrote then turns into NaN, and staging cannot overlap compute, so the
// output must match the normal build bit for bit.  The normal build compiles none
// of it.
#ifndef FA355_LDS_POISON
#define FA355_LDS_POISON 0
#endif
constexpr bool kLdsPoison = FA355_LDS_POISON != 0;

// Fills `bytes` (a multiple of 16) of LDS at `dst` with 0xff bytes, 16 per thread
// per pass, from the NT threads of the workgroup, and waits for the stores.
template <int NT>
__device__ __forceinline__ void lds_poison(char *dst, int bytes, int tid) {
    for (int off = tid * 16; off < bytes; off += NT * 16)
        *reinterpret_cast<u32x4_t *>(dst + off) = u32x4_t{~0u, ~0u, ~0u, ~0u};
    __builtin_amdgcn_s_waitcnt(0xc07f);     // lgkmcnt(0): the stores have landed
}

// ds_read_b64_tr_b16: each group of 16 lanes reads a 4-row x 16-column block of
// 16-bit values (lane L addresses 8 bytes of row (L % 16) / 4); lane L receives
// the four values of column L % 16, rows 0..3 in order.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t read_tr16(const char *p) {
#if defined(__HIP_DEVICE_COMPILE__)   // a gfx950 instruction: the host pass only sees a stub
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(p));
    return __builtin_bit_cast(u32x2_t, v);
#else
    (void)p;
    return u32x2_t{};
#endif
}

// V blocks sit in LDS unpadded, with the 16-byte chunks of each key row permuted:
// chunk c of row r is stored in slot c ^ v_swz(r).  The 32 lanes one transposed
// 8-byte read serves per LDS cycle (256 bytes) cover key rows 4g .. 4g + 3 and one
// 64-byte column group, chunks 4 nb .. 4 nb + 3; the XOR (bits 2-3 of the chunk index
// only) sends those four rows to four different 64-byte groups of banks.  A 128-byte
// row (head dim 64) shares its 64 banks with the next row, so there rows r and r + 2
// are the ones to separate.
template <int D>
__device__ __forceinline__ int v_swz(int r)
{
    return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
}

// Per-lane LDS offsets (from the start of a V block) of the transposed reads of the
// 32-column blocks nb = q + 4 m (q < 4; add 256 m bytes): lane L reads key row
// 4 (L / 32) + (L % 16) / 4 (+ 16 kstep, + 8), columns 16 ((L / 16) % 2) + 4 (L % 4)
// .. + 3 of the block, i.e. 8 bytes at chunk 4 nb + 2 ((L / 16) % 2) + (L % 4) / 2,
// byte 8 (L % 2) of that chunk.
template <int D>
__device__ __forceinline__ void v_read_offsets(int lane, int (&off)[(D / 32) < 4 ? (D / 32) : 4])
{
    const int r = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int sw4 = v_swz<D>(r) >> 2;
    const int base = r * 2 * D + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1);
#pragma unroll
    for (int q = 0; q < ((D / 32) < 4 ? (D / 32) : 4); ++q)
        off[q] = base + 64 * (q ^ sw4);
}

// A compile-time integer as a value (selects unrolled loop bodies).
template <int V> struct IntC { static constexpr int value = V; };

// Values of lanes L and L^32 (same query row), in a fixed order on both lanes.
__device__ __forceinline__ f32x2_t row_pair(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    f32x2_t r = {__uint_as_float(p[0]), __uint_as_float(p[1])};
    return r;
}

// Work-item order.  Workgroup w runs on XCD w % 8 (round-robin dispatch); the
// w-th workgroup of each XCD takes the next index of one contiguous range, so each
// XCD sees a contiguous slice of the logical order below.  The logical order cuts
// the B*Hq heads into groups of about B*Hq/8 consecutive heads (one group per XCD,
// so a group's K/V -- shared by consecutive GQA query heads -- stays in one L2),
// and walks each group query-tile-major: for causal attention the longest tiles of
// all the group's heads go first (longest-processing-time order), which lets the
// short tiles fill in the end of the launch evenly.
__device__ __forceinline__ void tile_of(int w, int total, int n_qtiles, int heads, bool causal,
                                        int &bh, int &qt) {
    const int xcd = w & 7, s = w >> 3;
    const int per = total >> 3, rem = total & 7;
    const int L = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + s;
    const int gh = heads >= 8 ? heads >> 3 : 1;          // heads per group
    const int full = (heads / gh) * gh * n_qtiles;       // tiles in whole groups
    int r, g0, gn;
    if (L < full) {
        const int g = L / (gh * n_qtiles);
        r = L - g * gh * n_qtiles;
        g0 = g * gh;
        gn = gh;
    } else {
        r = L - full;
        g0 = (heads / gh) * gh;
        gn = heads - g0;
    }
    const int rank = r / gn;
    bh = g0 + (r - rank * gn);
    qt = causal ? n_qtiles - 1 - rank : rank;
}

template <typename T, int D, int BC, int WAVES, bool CAUSAL, bool OUT_F32>
struct FwdTraits {
    static constexpr int BR = 32 * WAVES;
    static constexpr int NT = 64 * WAVES;
    static constexpr int DK = D / 16;            // 16-wide k chunks of Q K^T
    static constexpr int NB = D / 32;            // 32-wide output column blocks
    static constexpr int JB = BC / 32;           // 32-row blocks of the score tile
    static constexpr int KS = BC / 16;           // 16-key steps of P V
    static constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
    // K and V blocks go from global memory straight into LDS (no registers).
    // One 64-lane DMA instruction fills 64 consecutive 16-byte LDS slots, so a
    // block is laid out in slots: K row j takes CPR slots plus one pad slot (rows
    // start 4 banks apart: the 16 lanes one 16-byte read serves per LDS cycle, 16
    // consecutive rows at one chunk, hit 16 distinct groups of 4 banks); V row j
    // takes CPR slots, its chunks permuted by v_swz.  Pad slots, and slots past the
    // block, receive out-of-range (zero) loads.
    static constexpr int K_PITCH = D * 2 + 16;
    static constexpr int V_PITCH = D * 2;
    static constexpr int K_SLOTS = (BC * (CPR + 1) + 63) / 64 * 64;
    static constexpr int V_SLOTS = BC * CPR;
    static constexpr int K_INSTR = K_SLOTS / 64;
    static constexpr int N_INSTR = (K_SLOTS + V_SLOTS) / 64;   // DMA instructions per block
    static constexpr int P_INSTR = (N_INSTR + WAVES - 1) / WAVES;  // per wavefront
    static constexpr int K_STAGE = K_SLOTS * 16;
    static constexpr int V_STAGE = V_SLOTS * 16;
    static constexpr int STAGE = K_STAGE + V_STAGE;
    static constexpr int LDS = 2 * STAGE;
    static_assert(LDS == fwd_lds_bytes(D, BC), "LDS size");
    // Waves per SIMD to fit: two lets one wavefront's softmax run under the other's
    // matrix work; head dim 256 needs the whole register file for one (the
    // wavefront-pair kernel, fa_fwd_pair_kernel.hpp, splits that work).  At head dim
    // 64 the fp16 kernel (one row sum) fits four in the register file.
    static constexpr int OCC = (D <= 64 && WAVES == 4 && !Mfma<T>::kRoundedRowSum) ? 4
                             : (D <= 64 || (D == 128 && WAVES >= 4)) ? 2 : 1;
    static_assert(D % 32 == 0 && BC % 32 == 0, "tile shape");
    static_assert(BR * (BC / 8) % (64 * WAVES) == 0, "bias tile DMA: whole instructions per wave");
};

// SPLIT: the workgroup handles one of a.num_splits contiguous ranges of the tile's
// key/value blocks and writes its partial result, normalised by its own row sum,
// with its own lse, to a.o_part / a.lse_part; fa_fwd_merge_kernel combines them.
// BIAS: a 16-bit additive bias joins the scaled scores before the softmax (a bias
// of -inf masks the pair; a row left with no finite score gets O = 0, lse = -inf).
template <typename T, int D, int BC, int WAVES, bool CAUSAL, bool OUT_F32, bool SPLIT = false,
          bool BIAS = false>
__global__ void __launch_bounds__(64 * WAVES)
// The split and bias variants hold more per lane: at most two wavefronts per SIMD.
__attribute__((amdgpu_waves_per_eu((SPLIT || BIAS) && FwdTraits<T, D, BC, WAVES, CAUSAL, OUT_F32>::OCC > 2
                                       ? 2 : FwdTraits<T, D, BC, WAVES, CAUSAL, OUT_F32>::OCC)))
fa_fwd_kernel(FwdArgs a)
{
    using Tr = FwdTraits<T, D, BC, WAVES, CAUSAL, OUT_F32>;
    using M = Mfma<T>;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h2 = lane >> 5;

    int bh, qt, split = 0;
    if constexpr (SPLIT) {
        const int w = blockIdx.x / a.num_splits;
        split = blockIdx.x - w * a.num_splits;
        tile_of(w, a.total_tiles, a.n_qtiles, a.B * a.Hq, CAUSAL, bh, qt);
    } else {
        tile_of(blockIdx.x, a.total_tiles, a.n_qtiles, a.B * a.Hq, CAUSAL, bh, qt);
    }
    const int b = bh / a.Hq;
    const int hk = (bh - b * a.Hq) / a.group;
    const int N = a.N;
    const int i0 = qt * Tr::BR;
    const int iw0 = i0 + wave * 32;             // this wavefront's first query row
    const int iq = iw0 + l32;                   // this lane's query row
    constexpr int ROW = D * 2;                  // bytes per K/V/Q row
    const int head_bytes = N * ROW;

    const char *qh = static_cast<const char *>(a.q) + (size_t)bh * head_bytes;
    const char *kh = static_cast<const char *>(a.k) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const char *vh = static_cast<const char *>(a.v) + ((size_t)b * a.Hkv + hk) * head_bytes;

    // Q fragments: B operand of S^T = K Q^T.  Rows past N read as zero.
    u32x4_t qf[Tr::DK];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, head_bytes);
#pragma unroll
        for (int kk = 0; kk < Tr::DK; ++kk) {
            qf[kk] = load16(rq, iq * ROW + (kk * 16 + h2 * 8) * 2);
            qf[kk] ^= a.q_sign;
        }
    }

    const int kv_len = CAUSAL ? min(N, i0 + Tr::BR) : N;
    int t_begin = 0, n_kv = (kv_len + BC - 1) / BC;
    if constexpr (SPLIT) {
        // Split s takes blocks [s * chunk, (s + 1) * chunk) of the tile's range.
        const int chunk = (n_kv + a.num_splits - 1) / a.num_splits;
        t_begin = min(n_kv, split * chunk);
        n_kv = min(n_kv, t_begin + chunk);
    }

    // Per-lane source offsets of this wavefront's DMA instructions (loop-invariant):
    // instruction i = p * WAVES + wave fills slots 64 i .. 64 i + 63 of the stage.
    int dma_off[Tr::P_INSTR];
#pragma unroll
    for (int p = 0; p < Tr::P_INSTR; ++p) {
        const int i = p * WAVES + wave;
        if (i < Tr::K_INSTR) {
            const int slot = i * 64 + lane;
            const int row = slot / (Tr::CPR + 1), ch = slot - row * (Tr::CPR + 1);
            dma_off[p] = (row < BC && ch < Tr::CPR) ? row * ROW + ch * 16 : 0x7ffffff0;
        } else {
            const int slot = (i - Tr::K_INSTR) * 64 + lane;
            const int row = slot / Tr::CPR, sl = slot - row * Tr::CPR;
            dma_off[p] = row * ROW + 16 * (sl ^ v_swz<D>(row));
        }
    }

    // Block t of K and V into LDS stage `stage`.  The block's rows start each
    // buffer resource, so rows past N read as zero.
    // With a bias, each stage also holds the bias tile of the block: BR rows of BC
    // 16-bit values (BC * 2 bytes per row, rows contiguous), copied by the same DMA
    // path as K and V, so each bias row is fetched as whole 16-byte chunks.
    constexpr int B_CPR = BC / 8;                                   // chunks per row
    constexpr int B_INSTR = BIAS ? Tr::BR * B_CPR / 64 : 0;
    constexpr int STAGE = Tr::STAGE + (BIAS ? Tr::BR * BC * 2 : 0);
    // The two LDS stages are separate objects, and the loop below is unrolled by two
    // so that each access names its stage at compile time: the compiler can then
    // tell that reads of one stage do not alias the buffer-to-LDS copies landing in
    // the other, and does not make them wait for those copies.
    __shared__ __attribute__((aligned(16))) char lds0[STAGE];
    __shared__ __attribute__((aligned(16))) char lds1[STAGE];
    const char *bias_bh = nullptr;
    int bias_bytes = 0;
    if constexpr (BIAS) {
        const int h = bh - b * a.Hq;
        bias_bh = static_cast<const char *>(a.bias) + (b * a.bias_sb + h * a.bias_sh) * 2;
        // The extent of the (b, h) slice, rounded up to whole dwords: buffer range
        // checks zero any dword that is partly out of range, and the last valid key
        // may share a dword with the element after it (same dword, same page).
        bias_bytes = (int)((((long long)(N - 1) * a.bias_si + N) * 2 + 3) & ~3LL);
    }

    auto dma_block = [&](int t, char *st) {
        const int j0 = t * BC;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + (size_t)j0 * ROW, (N - j0) * ROW);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + (size_t)j0 * ROW, (N - j0) * ROW);
#pragma unroll
        for (int p = 0; p < Tr::P_INSTR; ++p) {
            const int i = p * WAVES + wave;
            if (Tr::N_INSTR % WAVES != 0 && i >= Tr::N_INSTR)
                break;
            dma16(i < Tr::K_INSTR ? rk : rv, st + i * 1024, dma_off[p]);
        }
        if constexpr (BIAS) {
            // Rows past N and keys past the (b, h) extent read as zero; keys past N
            // inside it are masked later anyway.
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias_bh, bias_bytes);
#pragma unroll
            for (int p = 0; p < B_INSTR / WAVES; ++p) {
                const int i = p * WAVES + wave;
                const int slot = i * 64 + lane;
                const int row = slot / B_CPR, ch = slot - row * B_CPR;
                const int off = (int)((long long)(i0 + row) * a.bias_si * 2) + j0 * 2 + ch * 16;
                dma16(rb, st + Tr::STAGE + i * 1024, i0 + row < N ? off : 0x7ffffff0);
            }
        }
    };

    // LDS read bases (per lane).  K: row l32, chunk h2 (16-byte reads).  V: the
    // transposed 64-bit read gives each 16-lane group a 4-key x 16-column block,
    // lane L receiving column L % 16 of it (v_read_offsets).
    const int k_rd = l32 * Tr::K_PITCH + h2 * 16;
    constexpr int VQ = Tr::NB < 4 ? Tr::NB : 4;
    int v_rd[VQ];
    v_read_offsets<D>(lane, v_rd);

    f32x16_t oacc[Tr::NB];
#pragma unroll
    for (int nb = 0; nb < Tr::NB; ++nb)
        oacc[nb] = f32x16_t{};
    float m_run = -__builtin_inff();
    float l_part = 0.0f;       // this lane's half of the row sum of rounded P
    float le_part = 0.0f;      // fp32 sum of unrounded P, for lse (bf16 only)
    // With a bias the scores are taken to log2 units (x = s c + bias log2 e) as
    // soon as they leave the matrix cores, and the multiplier below becomes 1.
    const float c = BIAS ? 1.0f : a.c;

    if (t_begin < n_kv) {
        if constexpr (kLdsPoison) {
            lds_poison<Tr::NT>(lds0, STAGE, tid);
            __syncthreads();
        }
        dma_block(t_begin, lds0);
    }
    __syncthreads();

    // Block t, held in stage S (block t + 1 goes to the other stage).
    auto iteration = [&](int t, auto stage) __attribute__((always_inline)) {
        constexpr int S = decltype(stage)::value;
        char *const cur = S == 0 ? lds0 : lds1;
        char *const nxt = S == 0 ? lds1 : lds0;
        const int j0 = t * BC;
        if (t + 1 < n_kv) {
            if constexpr (kLdsPoison) {
                lds_poison<Tr::NT>(nxt, STAGE, tid);
                __syncthreads();
            }
            dma_block(t + 1, nxt);
            if constexpr (kLdsPoison)
                __syncthreads();
        }

        // Blocks wholly above this wavefront's causal diagonal, and wavefronts
        // wholly past N, have nothing to add.
        const bool active = iw0 < N && (!CAUSAL || j0 <= iw0 + 31);
        if (active) {
            const char *kb = cur + k_rd;
            const char *vs = cur + Tr::K_STAGE;

            f32x16_t sacc[Tr::JB];
#pragma unroll
            for (int jb = 0; jb < Tr::JB; ++jb)
                sacc[jb] = f32x16_t{};
            // K fragments are read in batches of up to eight ahead of their matrix
            // instructions, so LDS latency overlaps the MFMA chain instead of
            // stalling each instruction.
            constexpr int KB = (8 / Tr::JB) < Tr::DK ? (8 / Tr::JB) : Tr::DK;   // kk per batch
#pragma unroll
            for (int k0 = 0; k0 < Tr::DK; k0 += KB) {
                u32x4_t kf[KB][Tr::JB];
#pragma unroll
                for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                    for (int jb = 0; jb < Tr::JB; ++jb)
                        kf[kk][jb] = *reinterpret_cast<const u32x4_t *>(
                            kb + jb * 32 * Tr::K_PITCH + (k0 + kk) * 32);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                    for (int jb = 0; jb < Tr::JB; ++jb)
                        sacc[jb] = M::run(kf[kk][jb], qf[k0 + kk], sacc[jb]);
            }

            if constexpr (BIAS) {
                // Lane L's keys j0 + 32 jb + 8 g + 4 (L/32) + 0..3 of its row: four
                // 16-bit values, one 8-byte LDS read.
                const char *bb = cur + Tr::STAGE +
                                 (wave * 32 + l32) * BC * 2;
#pragma unroll
                for (int jb = 0; jb < Tr::JB; ++jb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const u32x2_t w = *reinterpret_cast<const u32x2_t *>(
                            bb + (jb * 32 + 8 * g + 4 * h2) * 2);
                        float bv[4];
                        if constexpr (M::kSeparateLseSum) {        // bf16
                            bv[0] = __uint_as_float(w[0] << 16); bv[1] = __uint_as_float(w[0] & 0xffff0000u);
                            bv[2] = __uint_as_float(w[1] << 16); bv[3] = __uint_as_float(w[1] & 0xffff0000u);
                        } else {                                    // f16, one half at a time
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                bv[e] = (float)__builtin_bit_cast(
                                    _Float16, (uint16_t)(w[e >> 1] >> (16 * (e & 1))));
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sacc[jb][4 * g + e] = __builtin_fmaf(sacc[jb][4 * g + e], a.c,
                                                                 bv[e] * 1.44269504088896341f);
                    }
            }
            if ((CAUSAL && j0 + BC - 1 > iw0) || j0 + BC > N) {
#pragma unroll
                for (int jb = 0; jb < Tr::JB; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = j0 + jb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                        const bool vis = j < N && (!CAUSAL || j <= iq);
                        sacc[jb][r] = vis ? sacc[jb][r] : -__builtin_inff();
                    }
            }

            // Weights of this block against the row maximum estimate m, packed as
            // the B operand of P.V, with this lane's sums of them (rounded: lb;
            // unrounded, bf16 only: leb).
            u32x4_t pf[Tr::KS];
            float lb = 0.0f, leb = 0.0f;
            auto weights = [&](float m_sub) {
                lb = 0.0f;
                leb = 0.0f;
#pragma unroll
                for (int jb = 0; jb < Tr::JB; ++jb) {
                    float p[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[jb][r], c, -m_sub));
                        leb += p[r];
                    }
                    // The row sum adds the rounded weights the P.V product uses, so O
                    // is an exact weighted mean of V rows with those weights.
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t pk = M::pack(p[8 * s + 2 * e], p[8 * s + 2 * e + 1]);
                            pf[2 * jb + s][e] = pk;
                            if constexpr (M::kRoundedRowSum)
                                lb = M::sum2(pk, lb);
                        }
                }
            };

            // Any m gives the same O / l and m + log2 l, so the block maximum is only
            // needed when the weights against the current m could grow too large.
            // Once every row has a finite m, try the current m first: if this lane's
            // weights sum to at most kSumCap, each of them does too (they are >= 0),
            // and the block is done without a maximum.  A larger sum (or a non-finite
            // one) means the block raised the row maximum: take the block maximum,
            // rescale O and l to it and recompute the weights.
            bool fresh = (SPLIT || BIAS) ? __builtin_amdgcn_ballot_w64(m_run == -__builtin_inff()) == 0
                                         : t != t_begin;
            if (fresh) {
                weights(m_run);
                fresh = __builtin_amdgcn_ballot_w64(!(leb <= M::kSumCap)) == 0;
            }
            if (!fresh) {
                float mx = sacc[0][0];
#pragma unroll
                for (int jb = 0; jb < Tr::JB; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        mx = fmaxf(mx, sacc[jb][r]);
                const f32x2_t mp = row_pair(mx);
                const float m_new = fmaxf(m_run, fmaxf(mp[0], mp[1]) * c);
                // A row that has seen no finite score yet keeps m = -inf (possible
                // with a bias or a key-range split): nothing to scale, alpha = 1.
                const float alpha = ((SPLIT || BIAS) && m_new == -__builtin_inff())
                                        ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_part *= alpha;
                le_part *= alpha;
#pragma unroll
                for (int nb = 0; nb < Tr::NB; ++nb)
                    oacc[nb] *= alpha;
                m_run = m_new;
                // Rows still without a finite score subtract 0: their weights are
                // exp2(-inf) = 0, not NaN.
                weights(((SPLIT || BIAS) && m_run == -__builtin_inff()) ? 0.0f : m_run);
            }
            l_part += lb;
            le_part += leb;

#pragma unroll
            for (int nb = 0; nb < Tr::NB; ++nb) {
#pragma unroll
                for (int kstep = 0; kstep < Tr::KS; ++kstep) {
                    // Keys 16 kstep + 4 (L/32) + 0..3 and the same + 8 of column n.
                    const char *va = vs + v_rd[nb & 3] + 256 * (nb >> 2) + kstep * 16 * Tr::V_PITCH;
                    const u32x2_t lo = read_tr16(va), hi = read_tr16(va + 8 * Tr::V_PITCH);
                    const u32x4_t vf = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[nb] = M::run(vf, pf[kstep], oacc[nb]);
                }
            }
        }

        // The barrier's fence also waits for this iteration's DMA.
        __syncthreads();
    };
    for (int t = t_begin; t < n_kv; t += 2) {
        iteration(t, IntC<0>{});
        if (t + 1 < n_kv)
            iteration(t + 1, IntC<1>{});
    }

    // Epilogue: O = O / l, lse = ln2 * (m + log2 l).
    const f32x2_t ep = row_pair(le_part);
    const float le_tot = ep[0] + ep[1];
    float l_tot = le_tot;
    if constexpr (M::kRoundedRowSum) {
        const f32x2_t lp = row_pair(l_part);
        l_tot = lp[0] + lp[1];
    }
    if (SPLIT && iq < N) {
        // Rows that saw no key in this split: weight zero in the merge.
        const bool none = l_tot == 0.0f;
        const float inv = none ? 0.0f : 1.0f / l_tot;
        const size_t prow = (size_t)split * a.B * a.Hq * N + (size_t)bh * N + iq;
#pragma unroll
        for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4_t y = {oacc[nb][4 * g] * inv, oacc[nb][4 * g + 1] * inv,
                                   oacc[nb][4 * g + 2] * inv, oacc[nb][4 * g + 3] * inv};
                *reinterpret_cast<f32x4_t *>(a.o_part + prow * D + nb * 32 + 8 * g + 4 * h2) = y;
            }
        if (h2 == 0)
            a.lse_part[prow] = none ? -__builtin_inff() : kLn2 * (m_run + __log2f(le_tot));
    } else if (iq < N) {
        // With a bias a row can be left with no finite score: O = 0, lse = -inf.
        const bool none = BIAS && l_tot == 0.0f;
        const float inv = none ? 0.0f : 1.0f / l_tot;
        const size_t orow = ((size_t)bh * N + iq) * D;
#pragma unroll
        for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n0 = nb * 32 + 8 * g + 4 * h2;
                const float y0 = oacc[nb][4 * g + 0] * inv, y1 = oacc[nb][4 * g + 1] * inv;
                const float y2 = oacc[nb][4 * g + 2] * inv, y3 = oacc[nb][4 * g + 3] * inv;
                if constexpr (OUT_F32) {
                    f32x4_t y = {y0, y1, y2, y3};
                    *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.o) + orow + n0) = y;
                } else {
                    u32x2_t y = {M::pack(y0, y1), M::pack(y2, y3)};
                    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.o) + orow + n0) = y;
                }
            }
        if (h2 == 0 && a.lse)
            a.lse[(size_t)bh * N + iq] = none ? -__builtin_inff() : kLn2 * (m_run + __log2f(le_tot));
    }
}

// ---------------------------------------------------------------------------
// Split-KV merge: the partial results of one query row over disjoint key ranges
// combine exactly by the same rule as the online-softmax update ("MCU 上
// Transformer 模型的 Flash Attention 实现…", §二, merge equations), applied to
// normalised partials:  lse = log sum_s e^{lse_s},  O = sum_s e^{lse_s - lse} O_s.
// D/4 threads per row, four columns each.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) fa_fwd_merge_kernel(FwdArgs a)
{
    constexpr int TPR = D / 4;
    constexpr int RPB = 256 / TPR;
    const int64_t rows = (int64_t)a.B * a.Hq * a.N;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int col = (threadIdx.x % TPR) * 4;
    if (row >= rows)
        return;
    float m = -__builtin_inff();
    for (int s = 0; s < a.num_splits; ++s)
        m = fmaxf(m, a.lse_part[s * rows + row]);
    float wsum = 0.0f;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < a.num_splits; ++s) {
        const float ls = a.lse_part[s * rows + row];
        if (ls == -__builtin_inff())
            continue;
        const float w = __builtin_amdgcn_exp2f((ls - m) * 1.44269504088896341f);
        const f32x4_t x = *reinterpret_cast<const f32x4_t *>(a.o_part + (s * rows + row) * D + col);
        acc += w * x;
        wsum += w;
    }
    const float inv = 1.0f / wsum;
    const u32x2_t y = {Mfma<T>::pack(acc[0] * inv, acc[1] * inv), Mfma<T>::pack(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.o) + row * D + col) = y;
    if (col == 0 && a.lse)
        a.lse[row] = m + kLn2 * __log2f(wsum);
}

// ---------------------------------------------------------------------------
// fp32 inputs, head dim 64 (the small single-precision case): same algorithm on
// v_mfma_f32_32x32x2_f32, which takes one element per lane and so needs no
// transposed V: lane (n, half) reads V[j][n] straight from a row-major tile.
// P stays in fp32.  One LDS stage; this variant exists for exactness, not speed.
// ---------------------------------------------------------------------------
template <int WAVES, bool CAUSAL>
struct F32Traits {
    static constexpr int D = 64;
    static constexpr int BC = 32;
    static constexpr int BR = 32 * WAVES;
    static constexpr int NT = 64 * WAVES;
    static constexpr int KP = D + 1;             // padded K row (floats)
    static constexpr int K_FLOATS = BC * KP;
    static constexpr int V_FLOATS = BC * D;
    static constexpr int LDS = (K_FLOATS + V_FLOATS) * 4;
};

template <int WAVES, bool CAUSAL>
__global__ void __launch_bounds__(64 * WAVES)
fa_fwd_f32_kernel(FwdArgs a)
{
    using Tr = F32Traits<WAVES, CAUSAL>;
    constexpr int D = Tr::D, BC = Tr::BC;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float *kl = reinterpret_cast<float *>(smem);
    float *vl = kl + Tr::K_FLOATS;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h2 = lane >> 5;

    int bh, qt;
    tile_of(blockIdx.x, a.total_tiles, a.n_qtiles, a.B * a.Hq, CAUSAL, bh, qt);
    const int b = bh / a.Hq;
    const int hk = (bh - b * a.Hq) / a.group;
    const int N = a.N;
    const int i0 = qt * Tr::BR;
    const int iw0 = i0 + wave * 32;
    const int iq = iw0 + l32;
    const float *qh = static_cast<const float *>(a.q) + (size_t)bh * N * D;
    const float *kh = static_cast<const float *>(a.k) + ((size_t)b * a.Hkv + hk) * N * D;
    const float *vh = static_cast<const float *>(a.v) + ((size_t)b * a.Hkv + hk) * N * D;
    const float qsign = a.q_sign ? -1.0f : 1.0f;

    float qf[D / 2];
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk)
        qf[kk] = iq < N ? qsign * qh[(size_t)iq * D + 2 * kk + h2] : 0.0f;

    const int kv_len = CAUSAL ? min(N, i0 + Tr::BR) : N;
    const int n_kv = (kv_len + BC - 1) / BC;

    f32x16_t oacc[2] = {f32x16_t{}, f32x16_t{}};
    float m_run = -__builtin_inff();
    float l_part = 0.0f;
    const float c = a.c;

    for (int t = 0; t < n_kv; ++t) {
        const int j0 = t * BC;
        __syncthreads();
        if constexpr (kLdsPoison) {
            lds_poison<Tr::NT>(smem, Tr::LDS, tid);
            __syncthreads();
        }
        for (int x = tid; x < BC * D; x += Tr::NT) {
            const int row = x / D, col = x % D;
            const bool in = j0 + row < N;
            kl[row * Tr::KP + col] = in ? kh[(size_t)(j0 + row) * D + col] : 0.0f;
            vl[row * D + col] = in ? vh[(size_t)(j0 + row) * D + col] : 0.0f;
        }
        __syncthreads();

        const bool active = iw0 < N && (!CAUSAL || j0 <= iw0 + 31);
        if (!active)
            continue;

        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(kl[l32 * Tr::KP + 2 * kk + h2], qf[kk], s, 0, 0, 0);

        if ((CAUSAL && j0 + BC - 1 > iw0) || j0 + BC > N) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = j0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                const bool vis = j < N && (!CAUSAL || j <= iq);
                s[r] = vis ? s[r] : -__builtin_inff();
            }
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r)
            mx = fmaxf(mx, s[r]);
        const f32x2_t mp = row_pair(mx);
        const float mt = fmaxf(mp[0], mp[1]) * c;
        if (__builtin_amdgcn_ballot_w64(mt > m_run + kTau) != 0) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_part *= alpha;
            oacc[0] *= alpha;
            oacc[1] *= alpha;
            m_run = m_new;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m_run));
            l_part += p;
            const int j = 8 * (r >> 2) + 4 * h2 + (r & 3);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[j * D + nb * 32 + l32], p, oacc[nb], 0, 0, 0);
        }
    }

    const f32x2_t lp = row_pair(l_part);
    const float l_tot = lp[0] + lp[1];
    if (iq < N) {
        const float inv = 1.0f / l_tot;
        float *orow = static_cast<float *>(a.o) + ((size_t)bh * N + iq) * D;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4_t y = {oacc[nb][4 * g] * inv, oacc[nb][4 * g + 1] * inv,
                             oacc[nb][4 * g + 2] * inv, oacc[nb][4 * g + 3] * inv};
                *reinterpret_cast<f32x4_t *>(orow + nb * 32 + 8 * g + 4 * h2) = y;
            }
        if (h2 == 0 && a.lse)
            a.lse[(size_t)bh * N + iq] = kLn2 * (m_run + __log2f(l_tot));
    }
}

}  // namespace fa355
