// fa_fwd_pair_kernel.hpp -- the forward pass at head dimension 256 with two
// wavefronts per SIMD.
//
// At d = 256 one wavefront that owns 32 query rows holds 128 fp32 accumulators of
// O, 64 registers of Q fragments and the score tile: the whole register file, so
// only one wavefront fits on a SIMD and nothing runs under its softmax.  Here two
// wavefronts share the 32 rows and split the work of each 64-key block:
//
//   * wavefront h (h = 0, 1) of the pair computes the scores of keys 32h .. 32h+31
//     of the block (S^T = K Q^T over the full head dimension, 16 MFMAs) and their
//     weights against the row maximum estimate m ("MCU 上 Transformer 模型的 Flash
//     Attention 实现…", §二, online-softmax recurrence; the same lazy rescale as the
//     other 16-bit kernels);
//   * the two halves of P are exchanged through LDS, so that both hold P for all
//     64 keys;
//   * wavefront h accumulates output columns 128h .. 128h+127, O^T += V^T P^T
//     (16 MFMAs).
//
// Each wavefront then holds 64 output accumulators instead of 128, and the matrix
// work per wavefront and block is the same as the single-wavefront kernel's per
// half block.  The two wavefronts of a pair always use the same m: the rescale
// decision (a wavefront's weights summing past the cap, or the rows' first block)
// is taken per pair through an LDS flag, and the block maximum is combined across
// the pair through LDS.  The row sums of the two halves are added at the end.
//
// Workgroup: 8 wavefronts = 4 pairs = 128 query rows; K/V blocks of 64 rows in two
// LDS stages laid out as in fa_fwd_kernel (K rows padded by one 16-byte slot, V
// chunks XOR-swizzled), copied by buffer-to-LDS DMA.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa355 {

struct PairTraits {
    static constexpr int D = 256;
    static constexpr int BC = 64;
    static constexpr int WAVES = 8;
    static constexpr int NT = 64 * WAVES;
    static constexpr int BR = 128;                 // 4 pairs of 32 rows
    static constexpr int DK = D / 16;              // 16-wide k chunks of Q K^T
    static constexpr int NBH = D / 64;             // 32-wide output column blocks per wavefront
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
    static constexpr int PBUF = 4 * 4 * 64 * 16;   // P^T operands: 4 pairs x 4 key steps x 64 lanes
    static constexpr int MBUF = 4 * 2 * 32 * 4;    // one float per (pair, half, row)
    static constexpr int FLAGS = 2 * 4 * 4;        // rescale flags: [block parity][pair]
    static constexpr int LDS = 2 * STAGE + PBUF + 2 * MBUF + FLAGS;
    static_assert(STAGE == fwd_stage_bytes(D, BC) && LDS == fwd_pair_lds_bytes(), "LDS size");
};

template <typename T, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
fa_fwd_pair_kernel(FwdArgs a)
{
    using Tr = PairTraits;
    using M = Mfma<T>;
    constexpr int D = Tr::D, BC = Tr::BC;
    constexpr int ROW = D * 2;

    __shared__ __attribute__((aligned(16))) char lds0[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char lds1[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char pbuf[Tr::PBUF];
    __shared__ float mbuf[2][Tr::MBUF / 4];      // [0]: block maxima, [1]: final row sums
    __shared__ __attribute__((aligned(16))) int rescale_flag[2][4];   // [block parity][pair]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h2 = lane >> 5;
    const int g = wave >> 1;                    // pair: rows 32 g .. 32 g + 31 of the tile
    const int h = wave & 1;                     // keys 32 h .. of each block; columns 128 h ..

    int bh, qt;
    tile_of(blockIdx.x, a.total_tiles, a.n_qtiles, a.B * a.Hq, CAUSAL, bh, qt);
    const int b = bh / a.Hq;
    const int hk = (bh - b * a.Hq) / a.group;
    const int N = a.N;
    const int i0 = qt * Tr::BR;
    const int iw0 = i0 + g * 32;
    const int iq = iw0 + l32;
    const int head_bytes = N * ROW;
    const char *qh = static_cast<const char *>(a.q) + (size_t)bh * head_bytes;
    const char *kh = static_cast<const char *>(a.k) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const char *vh = static_cast<const char *>(a.v) + ((size_t)b * a.Hkv + hk) * head_bytes;

    // Q fragments of the pair's 32 rows over the whole head dimension.
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
    const int n_kv = (kv_len + BC - 1) / BC;

    // DMA source offsets, as in fa_fwd_kernel (instruction i = p * 8 + wave).
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

    // LDS read bases.  K: row 32 h + l32 of the block, chunk h2.  V: this
    // wavefront's column half (column blocks 4 h .. 4 h + 3; v_read_offsets).
    const int k_rd = (32 * h + l32) * Tr::K_PITCH + h2 * 16;
    int v_rd[4];
    v_read_offsets<D>(lane, v_rd);
    // P^T operand of key step s of pair g, lane `lane`.
    auto pslot = [&](int s) { return pbuf + ((g * 4 + s) * 64 + lane) * 16; };

    f32x16_t oacc[Tr::NBH];
#pragma unroll
    for (int nb = 0; nb < Tr::NBH; ++nb)
        oacc[nb] = f32x16_t{};
    float m_run = -__builtin_inff();
    float l_part = 0.0f;       // this lane's share of the row sum of rounded P (own keys)
    float le_part = 0.0f;      // fp32 sum of unrounded P, for lse (bf16 only)
    const float c = a.c;

    if (tid < 8)
        rescale_flag[tid >> 2][tid & 3] = 0;
    if (0 < n_kv) {
        if constexpr (kLdsPoison) {
            lds_poison<Tr::NT>(lds0, Tr::STAGE, tid);
            __syncthreads();
        }
        dma_block(0, lds0);
    }
    __syncthreads();

    auto iteration = [&](int t, auto stage) __attribute__((always_inline)) {
        constexpr int S = decltype(stage)::value;
        char *const cur = S == 0 ? lds0 : lds1;
        char *const nxt = S == 0 ? lds1 : lds0;
        const int j0 = t * BC;
        if (wave == 0 && lane < 4)
            rescale_flag[(t + 1) & 1][lane] = 0;     // read last in block t - 1
        if (t + 1 < n_kv) {
            if constexpr (kLdsPoison) {
                lds_poison<Tr::NT>(nxt, Tr::STAGE, tid);
                __syncthreads();
            }
            dma_block(t + 1, nxt);
            if constexpr (kLdsPoison)
                __syncthreads();
        }

        // Blocks wholly above the pair's causal diagonal, and pairs wholly past N,
        // have nothing to add (both wavefronts of a pair decide alike).
        const bool active = iw0 < N && (!CAUSAL || j0 <= iw0 + 31);
        f32x16_t sacc = f32x16_t{};
        // P^T operands: this wavefront's two key steps (keys 32 h .. 32 h + 31 of
        // the block) and the partner's two.
        u32x4_t pown[2], poth[2];
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
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t pk = M::pack(p[8 * s + 2 * e], p[8 * s + 2 * e + 1]);
                    pown[s][e] = pk;
                    if constexpr (M::kRoundedRowSum)
                        lb = M::sum2(pk, lb);
                }
        };
        auto publish = [&]() {
#pragma unroll
            for (int s = 0; s < 2; ++s)
                *reinterpret_cast<u32x4_t *>(pslot(2 * h + s)) = pown[s];
        };

        if (active) {
            const char *kb = cur + k_rd;
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
            const int jh = j0 + 32 * h;
            if ((CAUSAL && jh + 31 > iw0) || jh + 32 > N) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = jh + 8 * (r >> 2) + 4 * h2 + (r & 3);
                    const bool vis = j < N && (!CAUSAL || j <= iq);
                    sacc[r] = vis ? sacc[r] : -__builtin_inff();
                }
            }
            if (t != 0) {
                weights(m_run);
                if (__builtin_amdgcn_ballot_w64(!(leb <= M::kSumCap)) != 0 && lane == 0)
                    rescale_flag[t & 1][g] = 1;
                publish();
            }
        }
        __syncthreads();

        // A pair with a wavefront over the cap, and every pair in the rows' first
        // block, takes the block maximum (combined across the pair), rescales and
        // recomputes its weights.  The barriers this needs are taken by the whole
        // workgroup whenever any pair does it.
        const int *fl = rescale_flag[t & 1];
        const bool mine = t == 0 || fl[g] != 0;
        if (t == 0 || (fl[0] | fl[1] | fl[2] | fl[3]) != 0) {
            float mx = -__builtin_inff();
            if (active && mine) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, sacc[r]);
                const f32x2_t mp = row_pair(mx);
                mx = fmaxf(mp[0], mp[1]);
                if (h2 == 0)
                    mbuf[0][(g * 2 + h) * 32 + l32] = mx;
            }
            __syncthreads();
            if (active && mine) {
                const float mo = mbuf[0][(g * 2 + (h ^ 1)) * 32 + l32];
                const float m_new = fmaxf(m_run, fmaxf(mx, mo) * c);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_part *= alpha;
                le_part *= alpha;
#pragma unroll
                for (int nb = 0; nb < Tr::NBH; ++nb)
                    oacc[nb] *= alpha;
                m_run = m_new;
                weights(m_run);
                publish();
            }
            __syncthreads();
        }

        if (active) {
            l_part += lb;
            le_part += leb;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                poth[s] = *reinterpret_cast<const u32x4_t *>(pslot(2 * (h ^ 1) + s));
            // Column blocks 4 h .. 4 h + 3 of V; the own keys' rows first, then the
            // partner's (the order of the key steps is free).
            const char *vs = cur + Tr::K_STAGE + 256 * h;
            const char *vown = vs + 32 * h * Tr::V_PITCH;
            const char *voth = vs + 32 * (h ^ 1) * Tr::V_PITCH;
#pragma unroll
            for (int nb = 0; nb < Tr::NBH; ++nb) {
#pragma unroll
                for (int kstep = 0; kstep < 4; ++kstep) {
                    const char *va = (kstep < 2 ? vown : voth) + v_rd[nb] + (kstep & 1) * 16 * Tr::V_PITCH;
                    const u32x2_t lo = read_tr16(va), hi = read_tr16(va + 8 * Tr::V_PITCH);
                    const u32x4_t vf = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[nb] = M::run(vf, kstep < 2 ? pown[kstep & 1] : poth[kstep & 1], oacc[nb]);
                }
            }
        }

        // The barrier's fence also waits for this iteration's DMA.
        __syncthreads();
    };
    for (int t = 0; t < n_kv; t += 2) {
        iteration(t, IntC<0>{});
        if (t + 1 < n_kv)
            iteration(t + 1, IntC<1>{});
    }

    // Epilogue: the pair's row sums add up; O = O / l, lse = ln2 * (m + log2 l).
    const f32x2_t ep = row_pair(le_part);
    float le_own = ep[0] + ep[1];
    float l_own = le_own;
    if constexpr (M::kRoundedRowSum) {
        const f32x2_t lp = row_pair(l_part);
        l_own = lp[0] + lp[1];
    }
    if (h2 == 0) {
        mbuf[0][(g * 2 + h) * 32 + l32] = l_own;
        mbuf[1][(g * 2 + h) * 32 + l32] = le_own;
    }
    __syncthreads();
    const float l_oth = mbuf[0][(g * 2 + (h ^ 1)) * 32 + l32];
    const float le_oth = mbuf[1][(g * 2 + (h ^ 1)) * 32 + l32];
    // Both wavefronts add the same two numbers (in the same order), so they agree.
    const float l_tot = h == 0 ? l_own + l_oth : l_oth + l_own;
    const float le_tot = h == 0 ? le_own + le_oth : le_oth + le_own;
    if (iq < N) {
        const float inv = 1.0f / l_tot;
        const size_t orow = ((size_t)bh * N + iq) * D;
#pragma unroll
        for (int nb = 0; nb < Tr::NBH; ++nb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int n0 = 128 * h + nb * 32 + 8 * gg + 4 * h2;
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
        if (h == 0 && h2 == 0 && a.lse)
            a.lse[(size_t)bh * N + iq] = kLn2 * (m_run + __log2f(le_tot));
    }
}

}  // namespace fa355
