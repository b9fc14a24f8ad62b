// fa_decode_kernel.hpp -- attention of a few new queries against a long key/value
// cache, with the query heads of a grouped-query group packed into one wavefront.
//
// Decoding asks for Nq (a few) query rows per head against Nk cached keys.  A
// 32-row tile per query head would leave most MFMA rows empty, so the G = Hq/Hkv
// query heads that share a K/V head are packed together: one 64-lane wavefront
// carries all G*Nq (head, query) rows of a K/V group (the PackGQA scheme of
// "深度探索Flash-Attention中GQA性能调优技术解析", PackGQA section: the query heads of a
// group computed by one thread block, one warp serving several query heads).  In
// the [B, H, N, d] layout those rows are contiguous: row r of the group is query
// r % Nq of head hk*G + r / Nq, memory row (b*Hq + hk*G)*Nq + r.
//
// The key range is split into num_splits pieces (the num_splits parameter of the
// same page), one single-wavefront workgroup per (batch, K/V head, piece); each
// writes its normalised partial O and its lse, and fa_fwd_merge_kernel combines the
// pieces exactly (lse = log sum e^{lse_s}, O = sum e^{lse_s - lse} O_s).
//
// Per 32-key block the wavefront computes S^T = K Q^T and O^T += V^T P^T on the
// matrix cores as the square kernel does (fa_fwd_kernel.hpp documents the register
// layouts and the online softmax).  K fragments are loaded straight from global
// memory into registers, one block ahead; V goes through a two-stage LDS buffer
// (buffer-to-LDS DMA) for the transposed reads.  Loads for the block after next are
// always issued -- past the end they read zeros into a stage nobody reads -- so a
// fixed vmcnt wait separates the block being computed from the one in flight.
//
// Causal masking aligns the queries with the end of the cache: query i sees keys
// j <= i + Nk - Nq.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa355 {

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
fa_decode_kernel(DecodeArgs a)
{
    constexpr int BC = 32;
    constexpr int DK = D / 16, NB = D / 32, KS = BC / 16, CPR = D / 8;
    constexpr int ROW = D * 2;
    constexpr int V_PITCH = ROW + 32;                      // rows 8 banks apart
    constexpr int V_SLOTS = (BC * (CPR + 2) + 63) / 64 * 64;
    constexpr int V_INSTR = V_SLOTS / 64;
    constexpr int STAGE = V_SLOTS * 16;
    using M = Mfma<T>;
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int lane = threadIdx.x;
    const int l32 = lane & 31;
    const int h2 = lane >> 5;

    const int split = blockIdx.x % a.num_splits;
    const int bhk = blockIdx.x / a.num_splits;
    const int b = bhk / a.Hkv, hk = bhk - b * a.Hkv;
    const int Nk = a.Nk;
    const size_t row0 = ((size_t)b * a.Hq + (size_t)hk * a.group) * a.Nq;   // first packed row
    const int r = l32;                                     // this lane's packed row
    const int qi = r % a.Nq;                               // its query index
    const int jmax = CAUSAL ? qi + Nk - a.Nq : Nk - 1;      // last visible key
    const int j_all = CAUSAL ? Nk - a.Nq : Nk - 1;          // visible to every row

    // Q fragments of the packed rows; rows past group * Nq read as zero.
    u32x4_t qf[DK];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const char *>(a.q) + row0 * ROW,
                                                    a.rows * ROW);
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            qf[kk] = load16(rq, r * ROW + (kk * 16 + h2 * 8) * 2) ^ a.q_sign;
    }

    const int head_bytes = Nk * ROW;
    const char *kh = static_cast<const char *>(a.k) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const char *vh = static_cast<const char *>(a.v) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh, head_bytes);

    const int n_blk = (Nk + BC - 1) / BC;
    const int t_begin = min(n_blk, split * a.blocks_per_split);
    const int t_end = min(n_blk, t_begin + a.blocks_per_split);

    // V DMA source offsets within a block (rows of CPR chunks plus two pad slots).
    int v_src[V_INSTR];
#pragma unroll
    for (int p = 0; p < V_INSTR; ++p) {
        const int slot = p * 64 + lane;
        const int row = slot / (CPR + 2), ch = slot - row * (CPR + 2);
        v_src[p] = (row < BC && ch < CPR) ? row * ROW + ch * 16 : 0x7ffffff0;
    }
    // Loads of block t: K fragments into registers, V into LDS stage t & 1.  Block
    // offsets past the head read as zero (buffer range checks).
    auto load_k = [&](int t, u32x4_t (&kf)[DK]) {
        const int off = t * BC * ROW + l32 * ROW + h2 * 16;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            kf[kk] = load16(rk, off + kk * 32);
    };
    auto load_v = [&](int t) {
        char *st = smem + (t & 1) * STAGE;
        const int base = t * BC * ROW;
#pragma unroll
        for (int p = 0; p < V_INSTR; ++p)
            dma16(rv, st + p * 1024, v_src[p] == 0x7ffffff0 ? v_src[p] : base + v_src[p]);
    };
    // Waits until at most DK + V_INSTR vector memory operations are outstanding:
    // everything before the latest block's loads has landed.
    auto wait_previous = [&]() {
        constexpr int n = DK + V_INSTR;                    // < 64
        __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
    };

    const int v_rd = (4 * h2 + ((lane & 15) >> 2)) * V_PITCH + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

    f32x16_t oacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        oacc[nb] = f32x16_t{};
    float m_run = -__builtin_inff();
    float l_part = 0.0f, le_part = 0.0f;
    const float c = a.c;

    u32x4_t kf[DK];
    if (t_begin < t_end) {
        load_k(t_begin, kf);
        if constexpr (kLdsPoison)
            lds_poison<64>(smem + (t_begin & 1) * STAGE, STAGE, lane);
        load_v(t_begin);
    }
    for (int t = t_begin; t < t_end; ++t) {
        const int j0 = t * BC;
        u32x4_t kn[DK];
        load_k(t + 1, kn);                                 // past t_end: unused
        if constexpr (kLdsPoison)
            lds_poison<64>(smem + ((t + 1) & 1) * STAGE, STAGE, lane);
        load_v(t + 1);
        // The wait counts on the loads above being the latest ones issued.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kLdsPoison)
            __builtin_amdgcn_s_waitcnt(0);                 // every load has landed
        else
            wait_previous();                               // K(t) and V(t) have landed
        __builtin_amdgcn_sched_barrier(0);

        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            s = M::run(kf[kk], qf[kk], s);
        // Register q of lane L is key j0 + 8(q/4) + 4 h2 + q%4 of this lane's row.
        if (j0 + BC - 1 > j_all) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int j = j0 + 8 * (q >> 2) + 4 * h2 + (q & 3);
                s[q] = j <= jmax ? s[q] : -__builtin_inff();
            }
        }

        u32x4_t pf[KS];
        float lb = 0.0f, leb = 0.0f;
        auto weights = [&](float m_sub) {
            lb = 0.0f;
            leb = 0.0f;
            float p[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                p[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q], c, -m_sub));
                if constexpr (M::kSeparateLseSum)
                    leb += p[q];
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t pk = M::pack(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
                    pf[h][e] = pk;
                    lb = M::sum2(pk, lb);
                }
        };
        // As in the square kernel: accept the weights against the current m when no
        // lane's sum exceeds the cap; otherwise take the block maximum and rescale.
        // Rows without a finite score so far keep m = -inf and subtract 0.
        bool fresh = __builtin_amdgcn_ballot_w64(m_run == -__builtin_inff()) == 0;
        if (fresh) {
            weights(m_run);
            const float sum = M::kSeparateLseSum ? leb : lb;
            fresh = __builtin_amdgcn_ballot_w64(!(sum <= M::kSumCap)) == 0;
        }
        if (!fresh) {
            float mx = s[0];
#pragma unroll
            for (int q = 1; q < 16; ++q)
                mx = fmaxf(mx, s[q]);
            const f32x2_t mp = row_pair(mx);
            const float m_new = fmaxf(m_run, fmaxf(mp[0], mp[1]) * c);
            const float alpha = m_new == -__builtin_inff() ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_part *= alpha;
            le_part *= alpha;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                oacc[nb] *= alpha;
            m_run = m_new;
            weights(m_run == -__builtin_inff() ? 0.0f : m_run);
        }
        l_part += lb;
        le_part += leb;

        const char *vb = smem + (t & 1) * STAGE + v_rd;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const char *va = vb + ks * 16 * V_PITCH + nb * 64;
                const u32x2_t lo = read_tr16(va), hi = read_tr16(va + 8 * V_PITCH);
                const u32x4_t vf = {lo[0], lo[1], hi[0], hi[1]};
                oacc[nb] = M::run(vf, pf[ks], oacc[nb]);
            }
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            kf[kk] = kn[kk];
    }
    // Nothing may still be writing LDS when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(0);

    const f32x2_t lp = row_pair(l_part);
    const float l_tot = lp[0] + lp[1];
    float le_tot = l_tot;
    if constexpr (M::kSeparateLseSum) {
        const f32x2_t ep = row_pair(le_part);
        le_tot = ep[0] + ep[1];
    }
    if (r < a.rows) {
        // A row that saw no visible key in this piece has weight zero in the merge.
        const bool none = l_tot == 0.0f;
        const float inv = none ? 0.0f : 1.0f / l_tot;
        const size_t prow = (size_t)split * a.B * a.Hq * a.Nq + row0 + r;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4_t y = {oacc[nb][4 * g] * inv, oacc[nb][4 * g + 1] * inv,
                                   oacc[nb][4 * g + 2] * inv, oacc[nb][4 * g + 3] * inv};
                *reinterpret_cast<f32x4_t *>(a.o_part + prow * D + nb * 32 + 8 * g + 4 * h2) = y;
            }
        if (h2 == 0)
            a.lse_part[prow] = none ? -__builtin_inff() : kLn2 * (m_run + __log2f(le_tot));
    }
}

// ---------------------------------------------------------------------------
// Merge of the key-range pieces for few query rows (decoding has B*Hq*Nq of them,
// from a few dozen up): one workgroup per (row, 32 columns).  Each thread takes one
// piece's lse (there are at most 256 pieces), the workgroup forms the weights
// e^{lse_s - max} in LDS, groups of 8 threads (four columns each) weight their
// share of the pieces (loaded up front, with the lse values), and an LDS tree sums
// the groups.  Same rule as fa_fwd_merge_kernel:
// lse = log sum_s e^{lse_s},  O = sum_s e^{lse_s - lse} O_s.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) fa_decode_merge_kernel(FwdArgs a)
{
    constexpr int CW = 32;                     // columns per workgroup
    constexpr int TPR = CW / 4;                // threads per piece: four columns each
    constexpr int NG = 256 / TPR;              // groups of pieces
    __shared__ float wgt[256];
    __shared__ float red_m[4], red_w[4];
    __shared__ f32x4_t part[256];
    const int64_t rows = (int64_t)a.B * a.Hq * a.N;
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = a.num_splits;
    constexpr int PER = 256 / NG;              // pieces per thread at most (S <= 256)

    // This thread's partials are loaded together with the lse values, so the
    // merge waits on one round of memory reads, not two.
    const int col = blockIdx.y * CW + (tid % TPR) * 4, grp = tid / TPR;
    f32x4_t ov[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int s = grp + i * NG;
        ov[i] = s < S ? *reinterpret_cast<const f32x4_t *>(a.o_part + ((int64_t)s * rows + row) * D + col)
                      : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // The largest piece lse of the row.
    const float ls = tid < S ? a.lse_part[tid * rows + row] : -__builtin_inff();
    float m = ls;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0)
        red_m[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    // A piece that saw no key has lse -inf and a zero partial: weight 0.
    const float e = ls == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f((ls - m) * 1.44269504088896341f);
    wgt[tid] = e;
    float w = e;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        w += __shfl_xor(w, o);
    if (lane == 0)
        red_w[wave] = w;
    __syncthreads();

    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int s = grp + i * NG;
        if (s < S)
            acc += wgt[s] * ov[i];
    }
    part[tid] = acc;
    __syncthreads();
#pragma unroll
    for (int st = NG / 2; st > 0; st >>= 1) {
        if (grp < st)
            part[tid] += part[tid + st * TPR];
        __syncthreads();
    }
    if (tid < TPR) {
        const float wsum = (red_w[0] + red_w[1]) + (red_w[2] + red_w[3]);
        const float inv = 1.0f / wsum;
        const f32x4_t o = part[tid];
        const u32x2_t y = {Mfma<T>::pack(o[0] * inv, o[1] * inv), Mfma<T>::pack(o[2] * inv, o[3] * inv)};
        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.o) + row * D + col) = y;
        if (blockIdx.y == 0 && tid == 0 && a.lse)
            a.lse[row] = m + kLn2 * __log2f(wsum);
    }
}

}  // namespace fa355
