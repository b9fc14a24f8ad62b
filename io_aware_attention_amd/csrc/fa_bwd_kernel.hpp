// fa_bwd_kernel.hpp -- the backward pass of attention for gfx950: dQ, dK, dV from
// Q, K, V, O, dO and the forward pass's logsumexp, recomputing P tile by tile.
//
// The forward pass stores only O and lse, never the N x N score or probability
// matrix that standard attention keeps for the gradient computation
// ("FlashAttention 在昇腾 NPU 上是怎么省显存的？", section on the standard
// implementation's memory).  The backward pass rebuilds P from lse one tile at a
// time:  P_ij = exp(scale q_i.k_j - lse_i),  and applies the chain rule to
// O = softmax(scale Q K^T) V ("FlashAttention (VI)", equation Attention):
//
//   dV_j = sum_i P_ij dO_i           dP_ij = dO_i . V_j
//   dS_ij = P_ij (dP_ij - D_i),      D_i = sum_j P_ij dP_ij = dO_i . O_i
//   dQ_i = scale sum_j dS_ij K_j     dK_j = scale sum_i dS_ij Q_i
//
// Three kernels run in order on one stream:
//   fa_bwd_delta_kernel  D_i = dO_i . O_i into a caller-owned fp32 buffer;
//   fa_bwd_dkdv_role_kernel  one workgroup per (batch, K/V head, 128 keys) that
//                        walks every query block of every query head sharing the
//                        K/V head (GQA), so dK and dV need no atomics; two
//                        wavefronts per SIMD share 32 keys, one keeping K and
//                        dV in registers, the other V and dK;
//   fa_bwd_dq_kernel     one workgroup per (batch, query head, 256 or 128 queries):
//                        each wavefront keeps 32 queries' Q and dO fragments and
//                        dQ, and walks the key blocks; the wider workgroup shares
//                        each staged K/V block over more queries and is taken
//                        while it still gives every CU a workgroup.
// Matrix products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation;
// P and dS are rounded to the input type only as matrix operands.  Gradients are
// written in fp32.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa355 {

constexpr float kLog2e = 1.44269504088896341f;

// A compile-time step parity: loops unrolled by two name their LDS stage
// statically, so the stage being read is never the one the DMA engine fills.
template <int P> struct Parity { static constexpr int value = P; };

// A block of 32 rows of a [*, N, D] 16-bit tensor in LDS: each row takes D/8
// 16-byte slots plus PAD pad slots; DMA instructions fill 64 consecutive slots.
template <int D, int PAD>
struct RowBlock {
    static constexpr int CPR = D / 8;
    static constexpr int PITCH = (CPR + PAD) * 16;
    static constexpr int SLOTS = 32 * (CPR + PAD);
    static constexpr int INSTR = (SLOTS + 63) / 64;
    static constexpr int BYTES = INSTR * 1024;
};

// Rows j0 .. j0+31 of the tensor whose head starts at `head` (N rows of 2*D bytes)
// into LDS at `dst`; rows past N read as zero.  Wavefront `wave` of `waves` issues
// instructions wave, wave + waves, ...
template <int D, int PAD>
__device__ __forceinline__ void dma_rows(const char *head, int N, int j0, char *dst, int wave,
                                         int waves, int lane)
{
    using L = RowBlock<D, PAD>;
    constexpr int ROW = 2 * D;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(head + (size_t)j0 * ROW, (N - j0) * ROW);
    for (int i = wave; i < L::INSTR; i += waves) {
        const int slot = i * 64 + lane;
        const int row = slot / (L::CPR + PAD), ch = slot - row * (L::CPR + PAD);
        const int off = (row < 32 && ch < L::CPR) ? row * ROW + ch * 16 : 0x7ffffff0;
        dma16(r, dst + i * 1024, off);
    }
}

// A block of 32 rows of a [*, N, D] 16-bit tensor in LDS that is read both along
// its rows (16-byte fragments: 16 lanes read one chunk of 16 consecutive rows per
// LDS cycle) and across them (transposed 8-byte reads: 32 lanes read one 64-byte
// column group of 4 consecutive rows).  Rows are unpadded and chunk c of row r is
// stored in slot c ^ swz(r): for the row reads swz takes 16 different values over
// 16 consecutive rows (at D = 64, 8 over the 8 rows of one parity, the other
// parity using the other half of the banks), and its bits 2 and up send the 4 rows
// of a transposed read to 4 different 64-byte groups of banks, so neither pattern
// has bank conflicts.  Rows of 256 and 512 bytes (D = 128, 256) start on the same
// bank, so both take the same swz.
template <int D>
struct SwzBlock {
    static_assert(D == 64 || D == 128 || D == 256, "head dims of the backward pass");
    static constexpr int CPR = D / 8;
    static constexpr int PITCH = D * 2;
    static constexpr int INSTR = 32 * CPR / 64;
    static constexpr int BYTES = 32 * PITCH;
    static __device__ __forceinline__ int swz(int r) {
        return D == 64 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 3) : 4 * (r & 3) + ((r >> 2) & 3);
    }
};

// Rows j0 .. j0+31 into a SwzBlock at `dst` (rows past N read as zero).  Wavefront
// `wave` of `waves` issues instructions wave, wave + waves, ...
template <int D>
__device__ __forceinline__ void dma_rows_swz(const char *head, int N, int j0, char *dst, int wave,
                                             int waves, int lane)
{
    using L = SwzBlock<D>;
    constexpr int ROW = 2 * D;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(head + (size_t)j0 * ROW, (N - j0) * ROW);
    for (int i = wave; i < L::INSTR; i += waves) {
        const int slot = i * 64 + lane;
        const int row = slot / L::CPR, sl = slot - row * L::CPR;
        dma16(r, dst + i * 1024, row * ROW + 16 * (sl ^ L::swz(row)));
    }
}

// Per-lane byte offsets into a SwzBlock of the 16-byte row fragment (row L % 32,
// chunks 2 kk + L / 32): slot kk & 7, plus 256 bytes per 8 kk (the swizzle only
// permutes chunks within each 256-byte half of a 512-byte row), so head dim 256
// needs eight offsets, not sixteen.
template <int D>
constexpr int swz_row_slots() { return D / 16 < 8 ? D / 16 : 8; }
template <int D>
__device__ __forceinline__ void swz_row_offsets(int lane, int (&off)[swz_row_slots<D>()])
{
    using L = SwzBlock<D>;
    const int r = lane & 31, t = (lane >> 5) ^ L::swz(r);
#pragma unroll
    for (int kk = 0; kk < swz_row_slots<D>(); ++kk)
        off[kk] = r * L::PITCH + 16 * ((2 * kk) ^ t);
}
template <int D>
__device__ __forceinline__ int swz_row_at(const int (&off)[swz_row_slots<D>()], int kk)
{
    return off[kk & 7] + 256 * (kk >> 3);
}

// Per-lane byte offsets into a SwzBlock of the two transposed 8-byte reads that
// make up the A operand whose row is column n of 32-column block nb and whose
// k-slots are rows 16 ks + {0..3, 8..11} + 4 (L/32) -- the order in which
// pack_rows() lays out the B operand built from an accumulator (see the forward
// kernel's P.V product): [nb][0] for rows 0..3 (+ 4 (L/32)), [nb][1] for the rows
// 8 further on; add 16 ks rows (swz(r + 16) = swz(r), so the offsets carry over).
// Slot nb & 3, plus 256 bytes per 4 nb (as for the row reads).
template <int D>
constexpr int swz_tr_slots() { return D / 32 < 4 ? D / 32 : 4; }
template <int D>
__device__ __forceinline__ void swz_tr_offsets(int lane, int (&off)[swz_tr_slots<D>()][2])
{
    using L = SwzBlock<D>;
    const int r = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int j = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
        const int row = r + 8 * hi, f = L::swz(row);
#pragma unroll
        for (int nb = 0; nb < swz_tr_slots<D>(); ++nb)
            off[nb][hi] = row * L::PITCH + 16 * ((4 * nb + j) ^ f) + 8 * (lane & 1);
    }
}

// The transposed A operand of column block nb, key step ks from a SwzBlock.
template <int D>
__device__ __forceinline__ u32x4_t swz_tr_frag(const char *blk, const int (&off)[swz_tr_slots<D>()][2], int nb, int ks)
{
    const char *a = blk + ks * 16 * SwzBlock<D>::PITCH + 256 * (nb >> 2);
    const u32x2_t lo = read_tr16(a + off[nb & 3][0]), hi = read_tr16(a + off[nb & 3][1]);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// 32 fp32 values (one per row of a block) into LDS at `dst` (1 KB written; lanes
// past the 8 that carry data, and rows past N, write zeros).
__device__ __forceinline__ void dma_row_floats(const float *vec, int N, int j0, char *dst, int lane)
{
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vec + j0, (N - j0) * 4);
    dma16(r, dst, lane < 8 ? lane * 16 : 0x7ffffff0);
}

// An accumulator (rows 8*(r/4) + 4*(L/32) + r%4, column L%32) rounded to 16 bits
// as the B operand of a product over its rows (two 16-row k-steps).
template <typename T>
__device__ __forceinline__ void pack_rows(const float *x, u32x4_t out[2])
{
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            out[s][e] = Mfma<T>::pack(x[8 * s + 2 * e], x[8 * s + 2 * e + 1]);
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i.  D/8 lanes per row, 16 bytes each.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) fa_bwd_delta_kernel(BwdArgs a)
{
    constexpr int LPR = D / 8;                  // lanes per row
    constexpr int RPB = 256 / LPR;              // rows per block
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
    const int part = tid % LPR;
    const int64_t rows = (int64_t)a.B * a.Hq * a.N;
    float acc = 0.0f;
    if (row < rows) {
        const size_t at = (size_t)row * D + part * 8;
        if constexpr (Mfma<T>::kSeparateLseSum) {          // bf16: the high half of an fp32
            const u32x4_t g = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.dout) + at);
            const u32x4_t o = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.o) + at);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = __builtin_fmaf(__uint_as_float(g[e] << 16), __uint_as_float(o[e] << 16), acc);
                acc = __builtin_fmaf(__uint_as_float(g[e] & 0xffff0000u),
                                     __uint_as_float(o[e] & 0xffff0000u), acc);
            }
        } else {
            const f16x8_t g = *reinterpret_cast<const f16x8_t *>(static_cast<const _Float16 *>(a.dout) + at);
            const f16x8_t o = *reinterpret_cast<const f16x8_t *>(static_cast<const _Float16 *>(a.o) + at);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc = __builtin_fmaf((float)g[e], (float)o[e], acc);
        }
    }
#pragma unroll
    for (int w = 1; w < LPR; w <<= 1)
        acc += __shfl_xor(acc, w, LPR);
    if (row < rows && part == 0)
        a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV with two wavefronts per SIMD by role.  Workgroup: (batch, K/V head, 128
// keys) of eight wavefronts; wavefronts w and w + 4 (which share a SIMD) own the
// same 32 keys.  The first computes S = Q K^T and P for each 32-query block,
// accumulates dV^T += dO^T P and leaves P (fp32) in LDS; the second, one block
// behind, computes dP = dO V^T, dS = P * (dP - D) and accumulates dK^T += Q^T dS.
// Q, dO, lse and D blocks go through a ring of three LDS stages (the block being
// copied, the dV role's and the dK role's), P through three buffers; one barrier
// per block.  (At head dim 256 each role's fragments and accumulator slightly
// exceed half a SIMD's register file and some registers spill; two wavefronts per
// SIMD still beat one by 16 %.)
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
struct DkdvRoleTraits {
    static constexpr int BK = 128;
    static constexpr int DK = D / 16;
    static constexpr int NB = D / 32;
    using QL = SwzBlock<D>;
    static constexpr int Q_OFF = 0;
    static constexpr int G_OFF = QL::BYTES;
    static constexpr int L_OFF = 2 * QL::BYTES;        // lse of the block's 32 queries
    static constexpr int D_OFF = L_OFF + 1024;         // D of the block's 32 queries
    static constexpr int STAGE = D_OFF + 1024;
    static constexpr int PBUF = 4 * 64 * 16 * 4;       // P of the four key groups
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
fa_bwd_dkdv_role_kernel(BwdArgs a)
{
    using Tr = DkdvRoleTraits<T, D, CAUSAL>;
    using M = Mfma<T>;
    constexpr int ROW = 2 * D;
    __shared__ __attribute__((aligned(16))) char stage0[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char stage1[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char stage2[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char pbuf0[Tr::PBUF];
    __shared__ __attribute__((aligned(16))) char pbuf1[Tr::PBUF];
    __shared__ __attribute__((aligned(16))) char pbuf2[Tr::PBUF];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h2 = lane >> 5;
    const int kw = wave & 3;                    // the 32 keys this wavefront serves
    const bool dk_role = wave >= 4;

    // Key tile major: every head's first key tile, then every head's second, ...
    // With causal masking the first tiles see the most queries, so the longest
    // workgroups start first and the short ones fill the end of the launch.
    const int kt = blockIdx.x / (a.B * a.Hkv);
    const int bhk = blockIdx.x - kt * (a.B * a.Hkv);
    const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
    const int N = a.N;
    const int j0w = kt * Tr::BK + kw * 32;
    const int jk = j0w + l32;
    const int head_bytes = N * ROW;

    const char *kh = static_cast<const char *>(a.k) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const char *vh = static_cast<const char *>(a.v) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const float c = a.c;
    const int qb0 = CAUSAL ? (kt * Tr::BK) / 32 : 0;
    const int nqb = (N + 31) / 32;
    const int per_head = nqb - qb0;
    const int steps = per_head * a.group;

    int row_off[swz_row_slots<D>()], tr_off[swz_tr_slots<D>()][2];
    swz_row_offsets<D>(lane, row_off);
    swz_tr_offsets<D>(lane, tr_off);

    auto stage = [&](auto k) __attribute__((always_inline)) -> char * {
        constexpr int K = decltype(k)::value;
        return K == 0 ? stage0 : K == 1 ? stage1 : stage2;
    };
    auto pbuf = [&](auto k) __attribute__((always_inline)) -> char * {
        constexpr int K = decltype(k)::value;
        return K == 0 ? pbuf0 : K == 1 ? pbuf1 : pbuf2;
    };
    auto first_query = [&](int u) { return (qb0 + u % per_head) * 32; };
    auto load_step = [&](int u, char *st) {
        const int hq = hk * a.group + u / per_head;
        const int i0 = first_query(u);
        const size_t bh = (size_t)b * a.Hq + hq;
        if (wave < 2) {
            const char *base = static_cast<const char *>(wave == 0 ? a.q : a.dout) + bh * head_bytes;
            dma_rows_swz<D>(base, N, i0, st + (wave == 0 ? Tr::Q_OFF : Tr::G_OFF), 0, 1, lane);
        } else if (wave < 4) {
            const float *vec = (wave == 2 ? a.lse : a.delta) + bh * N;
            dma_row_floats(vec, N, i0, st + (wave == 2 ? Tr::L_OFF : Tr::D_OFF), lane);
        }
    };
    if (steps > 0) {
        if constexpr (kLdsPoison) {
            lds_poison<512>(stage0, Tr::STAGE, tid);
            __syncthreads();
        }
        load_step(0, stage0);
    }
    __syncthreads();

    // One role's whole loop and epilogue; the role is a compile-time constant so
    // each keeps only its own fragments and accumulators live.
    auto run_role = [&](auto role) __attribute__((always_inline)) {
        constexpr bool DKR = decltype(role)::value == 1;
        u32x4_t kv[Tr::DK];                     // K (dV role) or V (dK role) rows
        {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(DKR ? vh : kh, head_bytes);
            const uint32_t sign = DKR ? 0u : a.q_sign;
#pragma unroll
            for (int kk = 0; kk < Tr::DK; ++kk)
                kv[kk] = load16(r, jk * ROW + (kk * 16 + h2 * 8) * 2) ^ sign;
        }
        f32x16_t acc[Tr::NB];
#pragma unroll
        for (int nb = 0; nb < Tr::NB; ++nb)
            acc[nb] = f32x16_t{};

        // Iteration u: copy block u + 1 into stage (u + 1) % 3; the dV role takes
        // block u (stage and P buffer u % 3), the dK role block u - 1.
        auto iteration = [&](auto sidx, int u) __attribute__((always_inline)) {
            constexpr int S = decltype(sidx)::value;
            constexpr int SN = (S + 1) % 3, SP = (S + 2) % 3;
            if (u + 1 < steps) {
                if constexpr (kLdsPoison) {
                    lds_poison<512>(stage(IntC<SN>{}), Tr::STAGE, tid);
                    __syncthreads();
                }
                load_step(u + 1, stage(IntC<SN>{}));
                if constexpr (kLdsPoison)
                    __syncthreads();
            }
            const int ub = DKR ? u - 1 : u;
            const bool live = ub >= 0 && ub < steps;
            const int i0 = live ? first_query(ub) : 0;
            if (live && (!CAUSAL || i0 + 31 >= j0w)) {
                const char *st = DKR ? stage(IntC<SP>{}) : stage(IntC<S>{});
                char *pb = (DKR ? pbuf(IntC<SP>{}) : pbuf(IntC<S>{})) + kw * 4096 + lane * 16;
                const char *qb = st + Tr::Q_OFF, *gb = st + Tr::G_OFF;
                // S = Q K^T (dV role) or dP = dO V^T (dK role), 32 queries x 32 keys.
                f32x16_t s = f32x16_t{};
                const char *rb = DKR ? gb : qb;
#pragma unroll
                for (int kk = 0; kk < Tr::DK; ++kk)
                    s = M::run(*reinterpret_cast<const u32x4_t *>(rb + swz_row_at<D>(row_off, kk)), kv[kk], s);
                // Register r of lane L is query i0 + 8(r/4) + 4 h2 + r%4, key jk.
                float x[16];
                if constexpr (!DKR) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4_t lse4 = *reinterpret_cast<const f32x4_t *>(st + Tr::L_OFF + (8 * g + 4 * h2) * 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            x[4 * g + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + e], c, -lse4[e] * kLog2e));
                    }
                    // Only blocks on the causal diagonal or past N need the visibility test.
                    if ((CAUSAL && i0 < j0w + 31) || i0 + 32 > N || j0w + 32 > N) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int qi = i0 + 8 * (r / 4) + 4 * h2 + r % 4;
                            const bool vis = qi < N && jk < N && (!CAUSAL || jk <= qi);
                            x[r] = vis ? x[r] : 0.0f;
                        }
                    }
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<f32x4_t *>(pb + g * 1024) =
                            f32x4_t{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
                } else {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4_t p4 = *reinterpret_cast<const f32x4_t *>(pb + g * 1024);
                        const f32x4_t dl4 = *reinterpret_cast<const f32x4_t *>(st + Tr::D_OFF + (8 * g + 4 * h2) * 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            x[4 * g + e] = p4[e] * (s[4 * g + e] - dl4[e]);
                    }
                }
                u32x4_t px[2];
                pack_rows<T>(x, px);
                // dV^T += dO^T P (transposed dO) or dK^T += Q^T dS (transposed Q).
                const char *tb = DKR ? qb : gb;
#pragma unroll
                for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        acc[nb] = M::run(swz_tr_frag<D>(tb, tr_off, nb, ks), px[ks], acc[nb]);
            }
            // Its fence also waits for the copy of block u + 1 and the P writes.
            __syncthreads();
        };
        for (int u = 0; u <= steps; u += 3) {
            iteration(IntC<0>{}, u);
            if (u + 1 <= steps)
                iteration(IntC<1>{}, u + 1);
            if (u + 2 <= steps)
                iteration(IntC<2>{}, u + 2);
        }
        // Register r of lane L holds column 8(r/4) + 4 h2 + r%4 of block nb, key jk.
        if (jk < N) {
            const size_t row = ((size_t)b * a.Hkv + hk) * N + jk;
            float *out = DKR ? a.dk : a.dv;
            const float mul = DKR ? a.scale : 1.0f;
#pragma unroll
            for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n0 = nb * 32 + 8 * g + 4 * h2;
                    const f32x4_t y = {acc[nb][4 * g] * mul, acc[nb][4 * g + 1] * mul,
                                       acc[nb][4 * g + 2] * mul, acc[nb][4 * g + 3] * mul};
                    *reinterpret_cast<f32x4_t *>(out + row * D + n0) = y;
                }
        }
    };
    if (dk_role)
        run_role(IntC<1>{});
    else
        run_role(IntC<0>{});
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup: (batch, query head, 32 * WAVES queries); wavefront: 32 queries.
// Half the wavefronts stage K, the other half V, for every key block.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, int WAVES_>
struct DqTraits {
    static constexpr int WAVES = WAVES_;
    static constexpr int BR = 32 * WAVES;
    static constexpr int DK = D / 16;
    static constexpr int NB = D / 32;
    using KL = SwzBlock<D>;                    // K: row reads and transposed reads
    using VL = RowBlock<D, 1>;                 // V: row reads
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = KL::BYTES;
    static constexpr int STAGE = KL::BYTES + VL::BYTES;
};

template <typename T, int D, bool CAUSAL, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2)))
fa_bwd_dq_kernel(BwdArgs a)
{
    using Tr = DqTraits<T, D, CAUSAL, WAVES>;
    using M = Mfma<T>;
    using KL = typename Tr::KL;
    using VL = typename Tr::VL;
    constexpr int ROW = 2 * D;
    constexpr int BC = 32;
    __shared__ __attribute__((aligned(16))) char stage0[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char stage1[Tr::STAGE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int head_bytes = N * ROW;

    const char *kh = static_cast<const char *>(a.k) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const char *vh = static_cast<const char *>(a.v) + ((size_t)b * a.Hkv + hk) * head_bytes;
    u32x4_t qf[Tr::DK], gf[Tr::DK];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const char *>(a.q) + (size_t)bh * head_bytes, head_bytes);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(static_cast<const char *>(a.dout) + (size_t)bh * head_bytes, head_bytes);
#pragma unroll
        for (int kk = 0; kk < Tr::DK; ++kk) {
            qf[kk] = load16(rq, iq * ROW + (kk * 16 + h2 * 8) * 2) ^ a.q_sign;
            gf[kk] = load16(rg, iq * ROW + (kk * 16 + h2 * 8) * 2);
        }
    }
    // Rows past N: P = 0 (lse = +inf) and D = 0.
    const float lse2 = iq < N ? a.lse[(size_t)bh * N + iq] * kLog2e : __builtin_inff();
    const float dl = iq < N ? a.delta[(size_t)bh * N + iq] : 0.0f;
    const float c = a.c;

    f32x16_t dq[Tr::NB];
#pragma unroll
    for (int nb = 0; nb < Tr::NB; ++nb)
        dq[nb] = f32x16_t{};

    const int kv_len = CAUSAL ? min(N, i0 + Tr::BR) : N;
    const int n_kv = (kv_len + BC - 1) / BC;
    auto load_block = [&](int t, char *st) {
        constexpr int HALF = WAVES / 2;
        if (wave < HALF)
            dma_rows_swz<D>(kh, N, t * BC, st + Tr::K_OFF, wave, HALF, lane);
        else
            dma_rows<D, 1>(vh, N, t * BC, st + Tr::V_OFF, wave - HALF, HALF, lane);
    };

    int row_off[swz_row_slots<D>()], tr_off[swz_tr_slots<D>()][2];
    swz_row_offsets<D>(lane, row_off);
    swz_tr_offsets<D>(lane, tr_off);

    if constexpr (kLdsPoison) {
        lds_poison<64 * WAVES>(stage0, Tr::STAGE, tid);
        __syncthreads();
    }
    load_block(0, stage0);
    __syncthreads();

    auto step = [&](auto par, int t) {
        constexpr int P = decltype(par)::value;
        const char *st = P == 0 ? stage0 : stage1;
        if (t + 1 < n_kv) {
            if constexpr (kLdsPoison) {
                lds_poison<64 * WAVES>(P == 0 ? stage1 : stage0, Tr::STAGE, tid);
                __syncthreads();
            }
            load_block(t + 1, P == 0 ? stage1 : stage0);
            if constexpr (kLdsPoison)
                __syncthreads();
        }
        const int j0 = t * BC;
        if (iw0 < N && (!CAUSAL || j0 <= iw0 + 31)) {
            const char *kb = st + Tr::K_OFF, *vb = st + Tr::V_OFF;
            // S^T = K Q^T and dP^T = V dO^T (32 keys x 32 queries).
            f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
            for (int kk = 0; kk < Tr::DK; ++kk) {
                const u32x4_t ka = *reinterpret_cast<const u32x4_t *>(kb + swz_row_at<D>(row_off, kk));
                const u32x4_t va = *reinterpret_cast<const u32x4_t *>(vb + l32 * VL::PITCH + kk * 32 + h2 * 16);
                s = M::run(ka, qf[kk], s);
                dp = M::run(va, gf[kk], dp);
            }
            // Register r of lane L is key j0 + 8(r/4) + 4 h2 + r%4, query iq.  Only
            // blocks on the causal diagonal or past N need the visibility test.
            // (One test per block, outside the per-element loop: inside it the
            // compiler branches once per element.)
            float p[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
            if ((CAUSAL && j0 + 31 > iw0) || j0 + 32 > N) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = j0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                    const bool vis = j < N && (!CAUSAL || j <= iq);
                    p[r] = vis ? p[r] : 0.0f;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                ds[r] = p[r] * (dp[r] - dl);
            u32x4_t pd[2];
            pack_rows<T>(ds, pd);
            // dQ^T += K^T dS^T (transposed reads of K).
#pragma unroll
            for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    dq[nb] = M::run(swz_tr_frag<D>(kb, tr_off, nb, ks), pd[ks], dq[nb]);
        }
        __syncthreads();
    };
    for (int t = 0; t < n_kv; t += 2) {
        step(Parity<0>{}, t);
        if (t + 1 < n_kv)
            step(Parity<1>{}, t + 1);
    }

    if (iq < N) {
        const size_t row = (size_t)bh * N + iq;
#pragma unroll
        for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n0 = nb * 32 + 8 * g + 4 * h2;
                const f32x4_t y = {dq[nb][4 * g] * a.scale, dq[nb][4 * g + 1] * a.scale,
                                   dq[nb][4 * g + 2] * a.scale, dq[nb][4 * g + 3] * a.scale};
                *reinterpret_cast<f32x4_t *>(a.dq + row * D + n0) = y;
            }
    }
}

}  // namespace fa355
