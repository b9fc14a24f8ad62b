// fa_fwd_role_kernel.hpp -- the forward pass at head dimension 256 with the two
// wavefronts of each SIMD split by role.
//
// At d = 256 a wavefront that owns 32 query rows and does all of their work holds
// 128 fp32 accumulators of O, 64 registers of Q fragments and the score tile: the
// whole register file, so only one such wavefront fits on a SIMD and nothing runs
// under its softmax.  Here the work of each 32-row group is split between two
// wavefronts (w and w + 4 of the workgroup) by role:
//
//   * the score wavefront keeps Q and the running row maximum m.  For key block t
//     it computes S^T = K_t Q^T (16 MFMAs over the head dimension), the weights
//     P = exp2(S c - m) with the lazy rescale of the other 16-bit kernels ("MCU 上
//     Transformer 模型的 Flash Attention 实现…", §二, online-softmax recurrence),
//     the row sums, and leaves P, packed as the B operand of the P.V product, in
//     LDS -- with the factor e^(m_old - m_new) per row when m moved;
//   * the output wavefront keeps O.  One block behind, it scales O by that factor
//     when there is one and accumulates O^T += V_{t-1}^T P_{t-1}^T (16 MFMAs).
//
// Each of the two holds about half a register file, so both fit on one SIMD, and
// the score wavefront's exponentials run while the output wavefront's matrix
// products do.  K/V blocks of 32 keys go through a ring of three LDS stages (the
// block being copied, the score role's and the output role's; each laid out as
// in fa_fwd_kernel, K rows padded by one 16-byte slot, V chunks XOR-swizzled),
// P and the rescale factors through two buffers; one barrier per block.  At the
// end the score wavefront hands its row sums over through LDS, writes lse, and
// the output wavefront normalises and writes O.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa355 {

struct RoleTraits {
    static constexpr int D = 256;
    static constexpr int BC = 32;
    static constexpr int WAVES = 8;
    static constexpr int NT = 64 * WAVES;
    static constexpr int BR = 128;                 // four groups of 32 rows
    static constexpr int DK = D / 16;              // 16-wide k chunks of Q K^T
    static constexpr int NB = D / 32;              // 32-wide output column blocks
    static constexpr int KS = BC / 16;             // 16-key steps of P V
    static constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
    static constexpr int K_PITCH = D * 2 + 16;
    static constexpr int V_PITCH = D * 2;
    static constexpr int K_SLOTS = (BC * (CPR + 1) + 63) / 64 * 64;
    static constexpr int V_SLOTS = BC * CPR;
    static constexpr int K_INSTR = K_SLOTS / 64;
    static constexpr int N_INSTR = (K_SLOTS + V_SLOTS) / 64;
    static constexpr int P_INSTR = (N_INSTR + WAVES - 1) / WAVES;
    static constexpr int K_STAGE = K_SLOTS * 16;
    static constexpr int STAGE = K_STAGE + V_SLOTS * 16;
    static constexpr int PBUF = 2 * 4 * KS * 64 * 16;   // [parity][group][key step][lane]
    static constexpr int ABUF = 2 * 4 * 32 * 4;         // rescale factors [parity][group][row]
    static constexpr int FLAGS = 2 * 4 * 4;             // rescale flags [parity][group]
    static constexpr int LBUF = 4 * 32 * 4;             // final row sums [group][row]
    static constexpr int LDS = 3 * STAGE + PBUF + ABUF + FLAGS + LBUF;
    static_assert(STAGE == fwd_stage_bytes(D, BC) && LDS == fwd_role_lds_bytes(), "LDS size");
};

template <typename T, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
fa_fwd_role_kernel(FwdArgs a)
{
    using Tr = RoleTraits;
    using M = Mfma<T>;
    constexpr int D = Tr::D, BC = Tr::BC;
    constexpr int ROW = D * 2;

    __shared__ __attribute__((aligned(16))) char stage0[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char stage1[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char stage2[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char pbuf[Tr::PBUF];
    __shared__ float abuf[2][4][32];
    __shared__ int rflag[2][4];
    __shared__ float lbuf[4][32];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h2 = lane >> 5;
    // Wavefronts w and w + 4 share a SIMD (measured: pairing w with w ^ 1 instead
    // ran 8 % slower): w < 4 is group w's score role, w + 4 its output role.
    const int g = wave & 3;                     // rows 32 g .. 32 g + 31 of the tile
    const bool out_role = wave >= 4;

    int bh, qt;
    tile_of(blockIdx.x, a.total_tiles, a.n_qtiles, a.B * a.Hq, CAUSAL, bh, qt);
    const int b = bh / a.Hq;
    const int hk = (bh - b * a.Hq) / a.group;
    const int N = a.N;
    const int i0 = qt * Tr::BR;
    const int iw0 = i0 + g * 32;
    const int iq = iw0 + l32;
    const int head_bytes = N * ROW;
    const char *kh = static_cast<const char *>(a.k) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const char *vh = static_cast<const char *>(a.v) + ((size_t)b * a.Hkv + hk) * head_bytes;

    const int kv_len = CAUSAL ? min(N, i0 + Tr::BR) : N;
    const int n_kv = (kv_len + BC - 1) / BC;

    // DMA source offsets, as in fa_fwd_kernel (instruction i = p * 8 + wave): every
    // wavefront of both roles issues its share of each block's copy.
    int dma_off[Tr::P_INSTR];
#pragma unroll
    for (int p = 0; p < Tr::P_INSTR; ++p) {
        const int i = p * Tr::WAVES + wave;
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
    auto dma_block = [&](int t, char *st) {
        const int j0 = t * BC;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + (size_t)j0 * ROW, (N - j0) * ROW);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + (size_t)j0 * ROW, (N - j0) * ROW);
#pragma unroll
        for (int p = 0; p < Tr::P_INSTR; ++p) {
            const int i = p * Tr::WAVES + wave;
            if (Tr::N_INSTR % Tr::WAVES != 0 && i >= Tr::N_INSTR)
                break;
            dma16(i < Tr::K_INSTR ? rk : rv, st + i * 1024, dma_off[p]);
        }
    };
    auto stage = [&](auto k) __attribute__((always_inline)) -> char * {
        constexpr int K = decltype(k)::value;
        return K == 0 ? stage0 : K == 1 ? stage1 : stage2;
    };
    // Block t + 1 into the stage after t's, by every wavefront; in the debug build
    // the stage is poisoned first and the copy waited for.
    auto copy_next = [&](int t, char *st) __attribute__((always_inline)) {
        if (t + 1 < n_kv) {
            if constexpr (kLdsPoison) {
                lds_poison<Tr::NT>(st, Tr::STAGE, tid);
                __syncthreads();
            }
            dma_block(t + 1, st);
            if constexpr (kLdsPoison)
                __syncthreads();
        }
    };
    // Blocks wholly above the group's causal diagonal, and groups wholly past N,
    // have nothing to add (both roles of a group decide alike).
    auto active = [&](int t) { return iw0 < N && (!CAUSAL || t * BC <= iw0 + 31); };
    // P^T operand of key step s of group g in buffer `par`, lane `lane`.
    auto pslot = [&](int par, int s) { return pbuf + (((par * 4 + g) * Tr::KS + s) * 64 + lane) * 16; };

    if (n_kv > 0) {
        if constexpr (kLdsPoison) {
            lds_poison<Tr::NT>(stage0, Tr::STAGE, tid);
            __syncthreads();
        }
        dma_block(0, stage0);
    }
    __syncthreads();

    // Iteration t (t = 0 .. n_kv): block t + 1 is copied into stage (t + 1) % 3, the
    // score role takes block t (stage t % 3), the output role block t - 1.  Both
    // roles pass the same barriers.
    if (!out_role) {
        const char *qh = static_cast<const char *>(a.q) + (size_t)bh * head_bytes;
        u32x4_t qf[Tr::DK];
        {
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, head_bytes);
#pragma unroll
            for (int kk = 0; kk < Tr::DK; ++kk) {
                qf[kk] = load16(rq, iq * ROW + (kk * 16 + h2 * 8) * 2);
                qf[kk] ^= a.q_sign;
            }
        }
        const int k_rd = l32 * Tr::K_PITCH + h2 * 16;
        float m_run = -__builtin_inff();
        float l_part = 0.0f;       // this lane's half of the row sum of rounded P
        float le_part = 0.0f;      // fp32 sum of unrounded P, for lse (bf16 only)
        const float c = a.c;

        auto iteration = [&](int t, auto sidx) __attribute__((always_inline)) {
            constexpr int S = decltype(sidx)::value;
            copy_next(t, stage(IntC<(S + 1) % 3>{}));
            if (t < n_kv && active(t)) {
                const int j0 = t * BC;
                const char *kb = stage(IntC<S>{}) + k_rd;
                f32x16_t sacc = f32x16_t{};
                // K fragments in two batches of eight ahead of their matrix
                // instructions (all sixteen ahead, or two or four accumulator
                // chains, measured no faster).
#pragma unroll
                for (int k0 = 0; k0 < Tr::DK; k0 += 8) {
                    u32x4_t kf[8];
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk)
                        kf[kk] = *reinterpret_cast<const u32x4_t *>(kb + (k0 + kk) * 32);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk)
                        sacc = M::run(kf[kk], qf[k0 + kk], sacc);
                }
                if ((CAUSAL && j0 + BC - 1 > iw0) || j0 + BC > N) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = j0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                        const bool vis = j < N && (!CAUSAL || j <= iq);
                        sacc[r] = vis ? sacc[r] : -__builtin_inff();
                    }
                }

                u32x4_t pf[Tr::KS];
                float lb = 0.0f, leb = 0.0f;
                auto weights = [&](float m_sub) {
                    lb = 0.0f;
                    leb = 0.0f;
                    float p[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -m_sub));
                        leb += p[r];
                    }
                    // The row sum adds the rounded weights the P.V product uses.
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t pk = M::pack(p[8 * s + 2 * e], p[8 * s + 2 * e + 1]);
                            pf[s][e] = pk;
                            if constexpr (M::kRoundedRowSum)
                                lb = M::sum2(pk, lb);
                        }
                };
                // Any m gives the same O / l and m + log2 l while the weights stay in
                // range: after the first block, the current m is tried first, and the
                // block maximum is taken only if a lane's weights sum past the cap.
                bool fresh = t != 0;
                if (fresh) {
                    weights(m_run);
                    fresh = __builtin_amdgcn_ballot_w64(!(leb <= M::kSumCap)) == 0;
                }
                const int par = t & 1;
                if (!fresh) {
                    float mx = sacc[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r)
                        mx = fmaxf(mx, sacc[r]);
                    const f32x2_t mp = row_pair(mx);
                    const float m_new = fmaxf(m_run, fmaxf(mp[0], mp[1]) * c);
                    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                    l_part *= alpha;
                    le_part *= alpha;
                    m_run = m_new;
                    weights(m_run);
                    // The output role scales O by the same factor before it adds
                    // this block (O is still zero at the first block).
                    if (t != 0 && h2 == 0)
                        abuf[par][g][l32] = alpha;
                }
                if (lane == 0)
                    rflag[par][g] = (!fresh && t != 0) ? 1 : 0;
#pragma unroll
                for (int s = 0; s < Tr::KS; ++s)
                    *reinterpret_cast<u32x4_t *>(pslot(par, s)) = pf[s];
                l_part += lb;
                le_part += leb;
            }
            // Its fence also waits for the copy of block t + 1 and the P writes.
            __syncthreads();
        };
        for (int t = 0; t <= n_kv; t += 3) {
            iteration(t, IntC<0>{});
            if (t + 1 <= n_kv)
                iteration(t + 1, IntC<1>{});
            if (t + 2 <= n_kv)
                iteration(t + 2, IntC<2>{});
        }

        // Row sums to the output role; lse = ln2 * (m + log2 l).
        const f32x2_t ep = row_pair(le_part);
        const float le_tot = ep[0] + ep[1];
        float l_tot = le_tot;
        if constexpr (M::kRoundedRowSum) {
            const f32x2_t lp = row_pair(l_part);
            l_tot = lp[0] + lp[1];
        }
        if (h2 == 0)
            lbuf[g][l32] = l_tot;
        if (iq < N && h2 == 0 && a.lse)
            a.lse[(size_t)bh * N + iq] = kLn2 * (m_run + __log2f(le_tot));
        __syncthreads();
    } else {
        int v_rd[4];
        v_read_offsets<D>(lane, v_rd);
        f32x16_t oacc[Tr::NB];
#pragma unroll
        for (int nb = 0; nb < Tr::NB; ++nb)
            oacc[nb] = f32x16_t{};

        auto iteration = [&](int t, auto sidx) __attribute__((always_inline)) {
            constexpr int S = decltype(sidx)::value;
            copy_next(t, stage(IntC<(S + 1) % 3>{}));
            if (t >= 1 && active(t - 1)) {
                const int par = (t - 1) & 1;
                if (__builtin_amdgcn_readfirstlane(rflag[par][g]) != 0) {
                    const float al = abuf[par][g][l32];
#pragma unroll
                    for (int nb = 0; nb < Tr::NB; ++nb)
                        oacc[nb] *= al;
                }
                u32x4_t pf[Tr::KS];
#pragma unroll
                for (int s = 0; s < Tr::KS; ++s)
                    pf[s] = *reinterpret_cast<const u32x4_t *>(pslot(par, s));
                const char *vs = stage(IntC<(S + 2) % 3>{}) + Tr::K_STAGE;
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
            __syncthreads();
        };
        for (int t = 0; t <= n_kv; t += 3) {
            iteration(t, IntC<0>{});
            if (t + 1 <= n_kv)
                iteration(t + 1, IntC<1>{});
            if (t + 2 <= n_kv)
                iteration(t + 2, IntC<2>{});
        }

        __syncthreads();
        if (iq < N) {
            const float inv = 1.0f / lbuf[g][l32];
            const size_t orow = ((size_t)bh * N + iq) * D;
#pragma unroll
            for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    const int n0 = nb * 32 + 8 * gg + 4 * h2;
                    const float y0 = oacc[nb][4 * gg + 0] * inv, y1 = oacc[nb][4 * gg + 1] * inv;
                    const float y2 = oacc[nb][4 * gg + 2] * inv, y3 = oacc[nb][4 * gg + 3] * inv;
                    if constexpr (OUT_F32) {
                        f32x4_t y = {y0, y1, y2, y3};
                        *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.o) + orow + n0) = y;
                    } else {
                        u32x2_t y = {M::pack(y0, y1), M::pack(y2, y3)};
                        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.o) + orow + n0) = y;
                    }
                }
        }
    }
}

}  // namespace fa355
