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
//   fa_bwd_dkdv_kernel   one workgroup per (batch, K/V head, 128 keys): each
//                        wavefront keeps 32 keys' K and V fragments and their dK,
//                        dV accumulators in registers and walks every query block
//                        of every query head sharing the K/V head (GQA), so dK and
//                        dV need no atomics;
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

// 32 fp32 values (one per row of a block) into LDS at `dst` (1 KB written; lanes
// past the 8 that carry data, and rows past N, write zeros).
__device__ __forceinline__ void dma_row_floats(const float *vec, int N, int j0, char *dst, int lane)
{
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vec + j0, (N - j0) * 4);
    dma16(r, dst, lane < 8 ? lane * 16 : 0x7ffffff0);
}

// Transposed fragment of a row-major 16-bit block at pitch P (bytes): the A operand
// whose row is column n of 32-column block nb and whose k-slots are rows
// 16 ks + {0..3, 8..11} + 4 (L/32) -- the order in which pack_rows() lays out the
// B operand built from an accumulator (see the forward kernel's P.V product).
template <int P>
__device__ __forceinline__ u32x4_t tr_frag(const char *blk, int lane, int nb, int ks)
{
    const int off = (4 * (lane >> 5) + ((lane & 15) >> 2)) * P + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    const char *a = blk + off + ks * 16 * P + nb * 64;
    const u32x2_t lo = read_tr16(a), hi = read_tr16(a + 8 * P);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
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
// dK, dV.  Workgroup: (batch, K/V head, 128 keys); wavefront: 32 keys.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
struct DkdvTraits {
    static constexpr int WAVES = 4;
    static constexpr int BK = 32 * WAVES;
    static constexpr int DK = D / 16;
    static constexpr int NB = D / 32;
    using QL = RowBlock<D, 2>;                 // Q and dO blocks: row and transposed reads
    static constexpr int Q_OFF = 0;
    static constexpr int G_OFF = QL::BYTES;
    static constexpr int L_OFF = 2 * QL::BYTES;        // lse of the block's 32 queries
    static constexpr int D_OFF = L_OFF + 1024;         // D of the block's 32 queries
    static constexpr int STAGE = D_OFF + 1024;
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
fa_bwd_dkdv_kernel(BwdArgs a)
{
    using Tr = DkdvTraits<T, D, CAUSAL>;
    using M = Mfma<T>;
    using QL = typename Tr::QL;
    constexpr int ROW = 2 * D;
    __shared__ __attribute__((aligned(16))) char stage0[Tr::STAGE];
    __shared__ __attribute__((aligned(16))) char stage1[Tr::STAGE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h2 = lane >> 5;

    // Key tile major: every head's first key tile, then every head's second, ...
    // With causal masking the first tiles see the most queries, so the longest
    // workgroups start first and the short ones fill the end of the launch.
    const int kt = blockIdx.x / (a.B * a.Hkv);
    const int bhk = blockIdx.x - kt * (a.B * a.Hkv);
    const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
    const int N = a.N;
    const int j0w = kt * Tr::BK + wave * 32;   // this wavefront's first key
    const int jk = j0w + l32;                   // this lane's key (operand column)
    const int head_bytes = N * ROW;

    const char *kh = static_cast<const char *>(a.k) + ((size_t)b * a.Hkv + hk) * head_bytes;
    const char *vh = static_cast<const char *>(a.v) + ((size_t)b * a.Hkv + hk) * head_bytes;
    u32x4_t kf[Tr::DK], vf[Tr::DK];
    {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh, head_bytes), rv = make_rsrc(vh, head_bytes);
#pragma unroll
        for (int kk = 0; kk < Tr::DK; ++kk) {
            kf[kk] = load16(rk, jk * ROW + (kk * 16 + h2 * 8) * 2) ^ a.q_sign;
            vf[kk] = load16(rv, jk * ROW + (kk * 16 + h2 * 8) * 2);
        }
    }

    f32x16_t dk[Tr::NB], dv[Tr::NB];
#pragma unroll
    for (int nb = 0; nb < Tr::NB; ++nb) {
        dk[nb] = f32x16_t{};
        dv[nb] = f32x16_t{};
    }
    const float c = a.c;

    // Query blocks of 32: causal tiles start at the tile's first key.
    const int qb0 = CAUSAL ? (kt * Tr::BK) / 32 : 0;
    const int nqb = (N + 31) / 32;
    const int per_head = nqb - qb0;
    const int steps = per_head * a.group;

    auto load_step = [&](int u, char *st) {
        const int h = hk * a.group + u / per_head;
        const int i0 = (qb0 + u % per_head) * 32;
        const size_t bh = (size_t)b * a.Hq + h;
        if (wave < 2) {
            const char *base = static_cast<const char *>(wave == 0 ? a.q : a.dout) + bh * head_bytes;
            dma_rows<D, 2>(base, N, i0, st + (wave == 0 ? Tr::Q_OFF : Tr::G_OFF), 0, 1, lane);
        } else {
            const float *vec = (wave == 2 ? a.lse : a.delta) + bh * N;
            dma_row_floats(vec, N, i0, st + (wave == 2 ? Tr::L_OFF : Tr::D_OFF), lane);
        }
    };

    if (steps > 0) {
        if constexpr (kLdsPoison) {
            lds_poison<256>(stage0, Tr::STAGE, tid);
            __syncthreads();
        }
        load_step(0, stage0);
    }
    __syncthreads();

    auto step = [&](auto par, int u) {
        constexpr int P = decltype(par)::value;
        const char *st = P == 0 ? stage0 : stage1;
        if (u + 1 < steps) {
            if constexpr (kLdsPoison) {
                lds_poison<256>(P == 0 ? stage1 : stage0, Tr::STAGE, tid);
                __syncthreads();
            }
            load_step(u + 1, P == 0 ? stage1 : stage0);
            if constexpr (kLdsPoison)
                __syncthreads();
        }
        const int i0 = (qb0 + u % per_head) * 32;
        if (!CAUSAL || i0 + 31 >= j0w) {
            const char *qb = st + Tr::Q_OFF, *gb = st + Tr::G_OFF;
            // S = Q K^T and dP = dO V^T (32 queries x 32 keys): row reads of Q, dO.
            f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
            for (int kk = 0; kk < Tr::DK; ++kk) {
                const u32x4_t qa = *reinterpret_cast<const u32x4_t *>(qb + l32 * QL::PITCH + kk * 32 + h2 * 16);
                const u32x4_t ga = *reinterpret_cast<const u32x4_t *>(gb + l32 * QL::PITCH + kk * 32 + h2 * 16);
                s = M::run(qa, kf[kk], s);
                dp = M::run(ga, vf[kk], dp);
            }
            // Register r of lane L is query i0 + 8(r/4) + 4 h2 + r%4, key jk.  Only
            // blocks on the causal diagonal or past N need the visibility test.
            const bool edge = (CAUSAL && i0 < j0w + 31) || i0 + 32 > N || j0w + 32 > N;
            float p[16], ds[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4_t lse4 = *reinterpret_cast<const f32x4_t *>(st + Tr::L_OFF + (8 * g + 4 * h2) * 4);
                const f32x4_t dl4 = *reinterpret_cast<const f32x4_t *>(st + Tr::D_OFF + (8 * g + 4 * h2) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse4[e] * kLog2e));
                    if (edge) {
                        const int qi = i0 + 8 * g + 4 * h2 + e;
                        const bool vis = qi < N && jk < N && (!CAUSAL || jk <= qi);
                        p[r] = vis ? p[r] : 0.0f;
                    }
                    ds[r] = p[r] * (dp[r] - dl4[e]);
                }
            }
            u32x4_t pp[2], pd[2];
            pack_rows<T>(p, pp);
            pack_rows<T>(ds, pd);
            // dV^T += dO^T P and dK^T += Q^T dS (transposed reads of dO and Q).
#pragma unroll
            for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    dv[nb] = M::run(tr_frag<QL::PITCH>(gb, lane, nb, ks), pp[ks], dv[nb]);
                    dk[nb] = M::run(tr_frag<QL::PITCH>(qb, lane, nb, ks), pd[ks], dk[nb]);
                }
        }
        __syncthreads();      // its fence also waits for the next block's DMA
    };
    for (int u = 0; u < steps; u += 2) {
        step(Parity<0>{}, u);
        if (u + 1 < steps)
            step(Parity<1>{}, u + 1);
    }

    // Register r of lane L holds column 8(r/4) + 4 h2 + r%4 of block nb, key jk.
    if (jk < N) {
        const size_t row = ((size_t)b * a.Hkv + hk) * N + jk;
#pragma unroll
        for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n0 = nb * 32 + 8 * g + 4 * h2;
                const f32x4_t yk = {dk[nb][4 * g] * a.scale, dk[nb][4 * g + 1] * a.scale,
                                    dk[nb][4 * g + 2] * a.scale, dk[nb][4 * g + 3] * a.scale};
                const f32x4_t yv = {dv[nb][4 * g], dv[nb][4 * g + 1], dv[nb][4 * g + 2], dv[nb][4 * g + 3]};
                *reinterpret_cast<f32x4_t *>(a.dk + row * D + n0) = yk;
                *reinterpret_cast<f32x4_t *>(a.dv + row * D + n0) = yv;
            }
    }
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
    using KL = RowBlock<D, 2>;                 // K: row reads and transposed reads
    using VL = RowBlock<D, 1>;                 // V: row reads
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = KL::BYTES;
    static constexpr int STAGE = KL::BYTES + VL::BYTES;
};

template <typename T, int D, bool CAUSAL, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
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
            dma_rows<D, 2>(kh, N, t * BC, st + Tr::K_OFF, wave, HALF, lane);
        else
            dma_rows<D, 1>(vh, N, t * BC, st + Tr::V_OFF, wave - HALF, HALF, lane);
    };

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
                const u32x4_t ka = *reinterpret_cast<const u32x4_t *>(kb + l32 * KL::PITCH + kk * 32 + h2 * 16);
                const u32x4_t va = *reinterpret_cast<const u32x4_t *>(vb + l32 * VL::PITCH + kk * 32 + h2 * 16);
                s = M::run(ka, qf[kk], s);
                dp = M::run(va, gf[kk], dp);
            }
            // Register r of lane L is key j0 + 8(r/4) + 4 h2 + r%4, query iq.  Only
            // blocks on the causal diagonal or past N need the visibility test.
            const bool edge = (CAUSAL && j0 + 31 > iw0) || j0 + 32 > N;
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
                if (edge) {
                    const int j = j0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                    const bool vis = j < N && (!CAUSAL || j <= iq);
                    p = vis ? p : 0.0f;
                }
                ds[r] = p * (dp[r] - dl);
            }
            u32x4_t pd[2];
            pack_rows<T>(ds, pd);
            // dQ^T += K^T dS^T (transposed reads of K).
#pragma unroll
            for (int nb = 0; nb < Tr::NB; ++nb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    dq[nb] = M::run(tr_frag<KL::PITCH>(kb, lane, nb, ks), pd[ks], dq[nb]);
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
