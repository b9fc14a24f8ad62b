// fa_fp8_kernel.hpp -- FlashAttention forward with 8-bit floating-point inputs.
//
// Q, K and V are stored as OCP e4m3 codes (1 sign, 4 exponent bits with bias 7,
// 3 fraction bits, largest finite value 448), each tensor with one fp32 descale
// factor: the value of a stored element x is descale * e4m3(x).  This is the FP8
// variant of the forward pass that the GQA tuning page ("深度探索Flash-Attention中
// GQA性能调优技术解析", FP8 section) describes as halving the memory traffic, with
// the FP8 throughput figure of "FlashAttention (VI)", section on the evolution of
// the algorithm, FlashAttention-3.
// The function computed is the forward pass on the dequantised values:
//
//     O = softmax(scale * Qd Kd^T) Vd,   lse_i = log sum_j exp(scale * Qd_i . Kd_j),
//
// with O in bf16 and lse in fp32.
//
// The structure is that of the 16-bit kernel (fa_fwd_kernel.hpp): one workgroup per
// tile of 128 query rows, 64-key blocks of K and V streamed through two LDS stages by
// buffer-to-LDS DMA, each wavefront owning 32 query rows, the score tile computed
// transposed (S^T = K Q^T) so that each lane owns one query row.  What changes:
//
//  * Both products run on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32
//    accumulation): each lane supplies 32 bytes of A and 32 bytes of B, and the
//    instruction multiplies byte b of lane half h of A with byte b of lane half h
//    of B, so any byte order works as long as the two operands share it.  The
//    products of two e4m3 values are exact in fp32.
//  * The descales fold into the score multiplier (c = |scale| dq dk log2 e) and
//    into the output (times dv), so the matrix cores see the raw codes.
//  * P is rounded to e4m3 for P.V.  The kernel's weights are exp2(s c - m + 4),
//    m the row maximum estimate; the prescale by 2^4 keeps weights down to 2^-10 of
//    it in e4m3's normal range.  m is moved to the block maximum only when a lane's
//    weights sum to more than 448 (so that each stays within e4m3's range without
//    the maximum being taken in most blocks).  The row sum l adds the unrounded fp32
//    weights; O is normalised by it and the logsumexp is taken from it.
//  * V is not transposed in LDS: ds_read_b64_tr_b8 gives each 16-lane group an
//    8-key x 16-column block with lane L receiving column L % 16, so four reads
//    give a lane the 32 keys of its P bytes in the order of the score registers.
//  * K and V rows are 64 or 128 bytes with no padding; bank conflicts are avoided
//    by XOR-swizzling the 16-byte chunks within each row (the DMA source offsets
//    carry the permutation, so global reads stay whole 16-byte chunks).
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa355 {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// e4m3 x e4m3 -> fp32, 32 x 32 x 64, no block scaling.
__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ds_read_b64_tr_b8: each group of 16 lanes reads an 8-row x 16-byte block (lanes
// 2r and 2r+1 address the two 8-byte halves of row r); lane L receives byte L % 16
// of rows 0..7, row r in byte r of the result.
__device__ __forceinline__ i32x2_t read_tr8(const char *p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t *)(p));
#else
    (void)p;
    return i32x2_t{};
#endif
}

// Four fp32 values -> four e4m3 bytes (round to nearest even), first value lowest.
__device__ __forceinline__ int pack_fp8x4(float x0, float x1, float x2, float x3)
{
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, lo, true);
}

template <int D, int WAVES_ = 4>
struct Fp8Traits {
    static constexpr int WAVES = WAVES_;
    static constexpr int BR = 32 * WAVES;        // query rows per workgroup
    static constexpr int BC = 64;                // keys per block (the MFMA's k)
    static constexpr int NT = 64 * WAVES;
    static constexpr int KK = D / 64;            // 64-wide k steps of Q K^T
    static constexpr int NB = D / 32;            // 32-column output blocks
    static constexpr int CPR = D / 16;           // 16-byte chunks per row
    static constexpr int BLK = BC * D;           // bytes of one K or V block
    static constexpr int INSTR = 2 * BLK / 1024; // DMA instructions per block, K then V
    static constexpr int P_INSTR = INSTR / WAVES;
    static constexpr int STAGE = 2 * BLK;
    static constexpr int LDS = 2 * STAGE;
    static constexpr float PRE = 4.0f;           // log2 of the weights' prescale
    static constexpr float SUM_CAP = 448.0f;     // largest finite e4m3 value
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(INSTR % WAVES == 0, "whole DMA instructions per wavefront");

    // Chunk swizzles: chunk ch of row r sits in slot ch ^ swz(r) of the row.
    // K (16-byte reads, 16 lanes = 16 consecutive rows, one chunk column): the 16
    // (row, slot) pairs must cover 256 bytes.  V (transposed 8-byte reads, 32 lanes =
    // rows {0..3, 8..11} + const, two adjacent chunk columns): 8 rows x 2 slots.
    static __device__ __forceinline__ int k_swz(int r) { return D == 128 ? (r >> 1) & 7 : (r >> 2) & 3; }
    static __device__ __forceinline__ int v_swz(int r)
    {
        return D == 128 ? 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) : 2 * ((r >> 3) & 1);
    }
};

template <int D, bool CAUSAL, int WAVES = 4>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
fa_fwd_fp8_kernel(FwdArgs a)
{
    using Tr = Fp8Traits<D, WAVES>;
    constexpr int BC = Tr::BC;
    extern __shared__ __attribute__((aligned(16))) char smem[];

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
    const int head_bytes = N * D;

    const char *qh = static_cast<const char *>(a.q) + (size_t)bh * head_bytes;
    const char *kh = static_cast<const char *>(a.k) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const char *vh = static_cast<const char *>(a.v) + ((size_t)b * a.Hkv + hk) * head_bytes;

    // Q fragments (B operand of S^T = K Q^T): bytes 64 kk + 32 h2 .. +31 of row iq.
    i32x8_t qf[Tr::KK];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, head_bytes);
#pragma unroll
        for (int kk = 0; kk < Tr::KK; ++kk) {
            const u32x4_t x0 = load16(rq, iq * D + kk * 64 + h2 * 32) ^ a.q_sign;
            const u32x4_t x1 = load16(rq, iq * D + kk * 64 + h2 * 32 + 16) ^ a.q_sign;
            qf[kk] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                             (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
    }

    const int kv_len = CAUSAL ? min(N, i0 + Tr::BR) : N;
    const int n_kv = (kv_len + BC - 1) / BC;

    // DMA source offsets: instruction i = p * WAVES + wave fills slots 64 i' + lane
    // of the K block (i < INSTR / 2, i' = i) or the V block (i' = i - INSTR / 2).
    int dma_off[Tr::P_INSTR];
#pragma unroll
    for (int p = 0; p < Tr::P_INSTR; ++p) {
        const int i = p * Tr::WAVES + wave;
        const bool isk = i < Tr::INSTR / 2;
        const int s = (isk ? i : i - Tr::INSTR / 2) * 64 + lane;
        const int row = s / Tr::CPR, slot = s - row * Tr::CPR;
        const int ch = slot ^ (isk ? Tr::k_swz(row) : Tr::v_swz(row));
        dma_off[p] = row * D + ch * 16;
    }
    auto dma_block = [&](int t, int stage) {
        const int j0 = t * BC;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + (size_t)j0 * D, (N - j0) * D);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + (size_t)j0 * D, (N - j0) * D);
        char *st = smem + stage * Tr::STAGE;
#pragma unroll
        for (int p = 0; p < Tr::P_INSTR; ++p) {
            const int i = p * Tr::WAVES + wave;
            dma16(i < Tr::INSTR / 2 ? rk : rv, st + i * 1024, dma_off[p]);
        }
    };

    // LDS read offsets.  K: row 32 jb + l32, chunks 4 kk + 2 h2 + e (e = 0, 1).
    // V: key row 16 c + 4 h2 + (r % 4) + 8 (r / 4) for the group row r = (L % 16) / 2,
    // chunk 2 nb + (L / 16) % 2, half L % 2.
    int k_rd[Tr::KK][2];
    {
        const int sw = Tr::k_swz(l32);           // rows 32 jb + l32 share it
#pragma unroll
        for (int kk = 0; kk < Tr::KK; ++kk)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                k_rd[kk][e] = l32 * D + 16 * ((4 * kk + 2 * h2 + e) ^ sw);
    }
    int v_rd[Tr::NB];
    {
        const int r = (lane & 15) >> 1;
        const int key = 4 * h2 + (r & 3) + 8 * (r >> 2);   // + 16 c
        const int sw = Tr::v_swz(key);                      // independent of c
        const int g1 = (lane >> 4) & 1;
#pragma unroll
        for (int nb = 0; nb < Tr::NB; ++nb)
            v_rd[nb] = Tr::BLK + key * D + 16 * ((2 * nb + g1) ^ sw) + 8 * (lane & 1);
    }

    f32x16_t oacc[Tr::NB];
#pragma unroll
    for (int nb = 0; nb < Tr::NB; ++nb)
        oacc[nb] = f32x16_t{};
    float m_run = -__builtin_inff();
    float l_part = 0.0f;                       // this lane's half of the row sum
    const float c = a.c;

    if (n_kv > 0) {
        if constexpr (kLdsPoison) {
            lds_poison<Tr::NT>(smem, Tr::STAGE, tid);
            __syncthreads();
        }
        dma_block(0, 0);
    }
    __syncthreads();

    for (int t = 0; t < n_kv; ++t) {
        const int j0 = t * BC;
        if (t + 1 < n_kv) {
            if constexpr (kLdsPoison) {
                lds_poison<Tr::NT>(smem + ((t + 1) & 1) * Tr::STAGE, Tr::STAGE, tid);
                __syncthreads();
            }
            dma_block(t + 1, (t + 1) & 1);
            if constexpr (kLdsPoison)
                __syncthreads();
        }

        const bool active = iw0 < N && (!CAUSAL || j0 <= iw0 + 31);
        if (active) {
            const char *st = smem + (t & 1) * Tr::STAGE;

            f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
            i32x8_t kf[2][Tr::KK];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int kk = 0; kk < Tr::KK; ++kk) {
                    const u32x4_t x0 = *reinterpret_cast<const u32x4_t *>(st + k_rd[kk][0] + jb * 32 * D);
                    const u32x4_t x1 = *reinterpret_cast<const u32x4_t *>(st + k_rd[kk][1] + jb * 32 * D);
                    kf[jb][kk] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < Tr::KK; ++kk)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    sacc[jb] = mfma_fp8(kf[jb][kk], qf[kk], sacc[jb]);

            if ((CAUSAL && j0 + BC - 1 > iw0) || j0 + BC > N) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = j0 + jb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                        const bool vis = j < N && (!CAUSAL || j <= iq);
                        sacc[jb][r] = vis ? sacc[jb][r] : -__builtin_inff();
                    }
            }

            // Weights exp2(s c - (m - PRE)) against the row maximum estimate m,
            // packed as the B operand of P.V (byte 16 jb + r of the lane is score
            // register r of block jb), with this lane's sum of them.
            i32x8_t pf;
            float lb = 0.0f;
            auto weights = [&](float m_sub) {
                lb = 0.0f;
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float p[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[jb][4 * g + e], c, -m_sub));
                            lb += p[e];
                        }
                        pf[4 * jb + g] = pack_fp8x4(p[0], p[1], p[2], p[3]);
                    }
            };

            // O / l and m + log2 l do not depend on m, so the block maximum is only
            // taken when the weights against the current m could leave e4m3's range:
            // a lane sum of at most 448 bounds each weight by it.  After the first
            // block every row has a finite m.
            bool fresh = t != 0;
            if (fresh) {
                weights(m_run - Tr::PRE);
                fresh = __builtin_amdgcn_ballot_w64(!(lb <= Tr::SUM_CAP)) == 0;
            }
            if (!fresh) {
                float mx = sacc[0][0];
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        mx = fmaxf(mx, sacc[jb][r]);
                const f32x2_t mp = row_pair(mx);
                const float m_new = fmaxf(m_run, fmaxf(mp[0], mp[1]) * c);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_part *= alpha;
#pragma unroll
                for (int nb = 0; nb < Tr::NB; ++nb)
                    oacc[nb] *= alpha;
                m_run = m_new;
                weights(m_run - Tr::PRE);     // each weight <= 2^PRE
            }
            l_part += lb;

            // V^T fragments: read c gives bytes 8 c .. 8 c + 7, keys 16 c + 4 h2 +
            // {0..3, 8..11}: the keys of score registers 8 (c % 2) .. + 7 of block c / 2.
#pragma unroll
            for (int nb = 0; nb < Tr::NB; ++nb) {
                i32x8_t vf;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const i32x2_t x = read_tr8(st + v_rd[nb] + cc * 16 * D);
                    vf[2 * cc] = x[0];
                    vf[2 * cc + 1] = x[1];
                }
                oacc[nb] = mfma_fp8(vf, pf, oacc[nb]);
            }
        }

        // The barrier's fence also waits for this iteration's DMA.
        __syncthreads();
    }

    // Epilogue: O = dv * acc / l, lse = ln 2 * (m - PRE + log2 l).
    const f32x2_t lp = row_pair(l_part);
    const float l_tot = lp[0] + lp[1];
    if (iq < N) {
        const float inv = a.o_scale / l_tot;
        const size_t orow = ((size_t)bh * N + iq) * D;
#pragma unroll
        for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n0 = nb * 32 + 8 * g + 4 * h2;
                const u32x2_t y = {Mfma<BF16>::pack(oacc[nb][4 * g] * inv, oacc[nb][4 * g + 1] * inv),
                                   Mfma<BF16>::pack(oacc[nb][4 * g + 2] * inv, oacc[nb][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.o) + orow + n0) = y;
            }
        if (h2 == 0 && a.lse)
            a.lse[(size_t)bh * N + iq] = kLn2 * (m_run - Tr::PRE + __log2f(l_tot));
    }
}

template <int D, bool CAUSAL, int WAVES = 4>
hipError_t launch_fwd_fp8_impl(const FwdArgs &a, hipStream_t stream)
{
    using Tr = Fp8Traits<D, WAVES>;
    const void *fn = reinterpret_cast<const void *>(&fa_fwd_fp8_kernel<D, CAUSAL, WAVES>);
    FwdArgs arg = a;
    void *params[] = {&arg};
    return hipLaunchKernel(fn, dim3(a.total_tiles), dim3(Tr::NT), params, Tr::LDS, stream);
}

}  // namespace fa355
