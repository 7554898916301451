// DIFF V1 backward on bf16 MFMA (gfx950): d = 64 per map, dv = 128, optional RMSNorm epilogue.
//
// Gradients of y = (1 - lambda_init) w * o / rms(o), o = A1 V - lambda A2 V, A_k = softmax(s Q_k K_k^T)
// ("Differential Transformer: Noise-Canceling Attention by Subtraction", sections "The mechanism"
// and "Making lambda learnable and stable"), by the chain rule:
//   RMSNorm:  u = o / r, du = (1 - lambda_init) w * dy,  go = dL/do = (du - u mean(du u)) / r,
//             dL/dw = sum over rows of dy (1 - lambda_init) u
//   maps:     dP = go V^T (shared by both maps), D_k = go . (A_k V) per row,
//             dS1 = A1 (dP - D1),  dS2 = -lambda A2 (dP - D2),
//             dQ_k = s dS_k K_k,  dK_k = s dS_k^T Q_k,  dV = (A1 - lambda A2)^T go,
//             dlambda = -sum over rows of D2.
// The forward's training outputs supply each map's log-sum-exp (so A_k is recomputed exactly
// from the scores) and A_k V (for D_k and o).
//
// Kernels (no atomics; every sum is taken in a fixed order):
//  - bwd_pre: half a wave per row: o, go (stored bf16 as an MFMA operand), D1, D2, and per-block
//    partial sums of dL/dw and dlambda.
//  - bwd_dq: query-tile parallel like the forward (S^T = K Q^T, lane = query): K1, K2, V tiles of
//    32 keys staged through LDS, one block barrier per pair of tiles; dP^T = V go^T;
//    dQ_k^T += K_k^T dS_k^T with K^T read by the transposing LDS read.
//  - bwd_dkdv: key-tile parallel (S = Q K^T, lane = key): each lane keeps its key's K1, K2, V rows
//    in registers and the block walks the query tiles (Q1, Q2, go staged through LDS);
//    dV^T += go^T (A1 - lambda A2) and dK_k^T += Q_k^T dS_k with the transposed operands again
//    read by ds_read_b64_tr_b16. Query tiles come in pairs, one block barrier per pair; where the
//    pair holds no masked (query, key) pair for any wave of the block, its 64 MFMAs run in a fixed
//    order with the second tile's score MFMAs beside the first tile's vector work and the first
//    tile's gradient MFMAs beside the second tile's, each operand read issued four MFMAs ahead.
// Tiles that hold no masked (query, key) pair skip the per-element visibility test.
//  - bwd_reduce: dlambda per head and dL/dw per channel from the partials.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_tile.hpp"
#include "bwd_tile.hpp"

namespace diffattn {

namespace {

using namespace bwdt;

constexpr int kD = 64;
constexpr int kDV = 128;
constexpr int kKTile = kBN * kD * 2;    // bytes of one 32-row, 64-wide tile
constexpr int kVTile = kBN * kDV * 2;   // bytes of one 32-row, 128-wide tile
constexpr int kPreRows = 64;            // rows per bwd_pre block (4 waves x 16 rows)
// dK/dV query-tile stage: Q1 | Q2 (64 wide) | go (128 wide) | lse [32][2] | dd [32][2]
constexpr int kQStats = 2 * kKTile + kVTile;
constexpr int kQStage = kQStats + 2 * kBN * 2 * 4;
constexpr int kQStages = 4;
constexpr int kKStage = 2 * kKTile + kVTile;   // dQ key-tile stage: K1 | K2 (64 wide) | V
constexpr int kKStages = 4;                      // dQ ring: two pairs of key tiles

__device__ __forceinline__ int rowop_b(int row, int kk, int h2) { return rowop<kD>(row, kk, h2); }
__device__ __forceinline__ int trop_b(int lane, int kb, int mt, int hi) { return trop<kD>(lane, kb, mt, hi); }
__device__ __forceinline__ int rowop_v(int row, int kk, int h2) { return rowop<kDV>(row, kk, h2); }
__device__ __forceinline__ int trop_v(int lane, int kb, int ct, int hi) { return trop<kDV>(lane, kb, ct, hi); }

// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // a wave takes its rows two at a time: lanes 0-31 one row, lanes 32-63 the next, each lane
    // the four channels c0 .. c0 + 3 (16-byte map loads, 8-byte dout loads and go stores)
    const int hl = lane >> 5, c0 = 4 * (lane & 31);
    const float lam = a.lam[h];
    const float kappa = 1.f - a.lambda_init;
    float w[4] = {1.f, 1.f, 1.f, 1.f};
    if (a.epi && a.norm_w)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = a.norm_w[c0 + j];
    float gw[4] = {0.f, 0.f, 0.f, 0.f}, glam = 0.f;   // partial dL/dw (4 channels) and dlambda
    // steps of two rows in chunks of two steps: a chunk's loads are issued while the previous
    // chunk is reduced (rows past the end read row 0 and are not used)
    constexpr int R = kPreRows / 4, CH = 2, NC = R / (2 * CH);
    struct Chunk { f32x4 a1[CH], a2[CH]; bf16x4 dy[CH]; };
    auto row_of = [&](int c, int k) { return blk * kPreRows + wave * R + 2 * (c * CH + k) + hl; };
    auto load_chunk = [&](int c, Chunk& r) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int i = row_of(c, k);
            const int ii = i < a.seq_q ? i : 0;
            const float* mp = a.maps + (((int64_t)b * a.seq_q + ii) * a.heads + h) * 2 * kDV;
            r.a1[k] = *(const f32x4*)(mp + c0);
            r.a2[k] = *(const f32x4*)(mp + kDV + c0);
            const bf16* dyp = (const bf16*)a.dout + b * a.dos[0] + (int64_t)ii * a.dos[1] + (int64_t)h * a.dos[2];
            r.dy[k] = *(const bf16x4*)(dyp + c0);
        }
    };
    auto reduce_chunk = [&](int c, const Chunk& r) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int i = row_of(c, k);
            const bool ok = i < a.seq_q;   // the half-wave sums run on every lane; only valid rows count
            float dy[4], g[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) dy[j] = (float)r.dy[k][j];
            if (a.epi) {
                float o[4];
                {
#pragma clang fp contract(off)
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = r.a1[k][j] - lam * r.a2[k][j];
                }
                const float ms = half_sum((o[0] * o[0] + o[1] * o[1]) + (o[2] * o[2] + o[3] * o[3])) * (1.f / kDV);
                const float inv = 1.f / sqrtf(ms + a.eps);
                float u[4], du[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u[j] = o[j] * inv;
                    du[j] = kappa * w[j] * dy[j];
                }
                const float t = half_sum((du[0] * u[0] + du[1] * u[1]) + (du[2] * u[2] + du[3] * u[3])) * (1.f / kDV);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    g[j] = (du[j] - u[j] * t) * inv;
                    if (ok) gw[j] += dy[j] * kappa * u[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) g[j] = dy[j];
            }
            // dlambda takes go in fp32; go enters the MFMA kernels rounded to bf16, and D_k takes the
            // same rounded values, so that each row of dS_k sums to zero as the softmax Jacobian's do
            const float gl = half_sum((g[0] * r.a2[k][0] + g[1] * r.a2[k][1]) + (g[2] * r.a2[k][2] + g[3] * r.a2[k][3]));
            if (ok) glam -= gl;
            bf16x4 gb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gb[j] = (bf16)g[j];
                g[j] = (float)gb[j];
            }
            const float D1 = half_sum((g[0] * r.a1[k][0] + g[1] * r.a1[k][1]) + (g[2] * r.a1[k][2] + g[3] * r.a1[k][3]));
            const float D2 = half_sum((g[0] * r.a2[k][0] + g[1] * r.a2[k][1]) + (g[2] * r.a2[k][2] + g[3] * r.a2[k][3]));
            if (ok) {
                const int64_t row = ((int64_t)b * a.heads + h) * a.seq_q + i;
                *(bf16x4*)(a.go + row * kDV + c0) = gb;
                if ((lane & 31) == 0) *(float2*)(a.dd + 2 * row) = make_float2(D1, D2);
            }
        }
    };
    Chunk buf[2];
    load_chunk(0, buf[0]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c + 1 < NC) load_chunk(c + 1, buf[(c + 1) & 1]);
        reduce_chunk(c, buf[c & 1]);
    }
    // block partials in a fixed order: the two halves of each wave, then waves 0..3
    __shared__ float sw[4][kDV];
    __shared__ float sl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) gw[j] = sum_halves(gw[j]);
    glam = sum_halves(glam);
    if (hl == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j) sw[wave][c0 + j] = gw[j];
    if (lane == 0) sl[wave] = glam;
    __syncthreads();
    const int64_t pb = ((int64_t)b * a.heads + h) * gridDim.x + blk;   // partial index
    if (tid < kDV && a.epi) {
        const float s = ((sw[0][tid] + sw[1][tid]) + sw[2][tid]) + sw[3][tid];
        a.wpart[(int64_t)tid * a.n_part + pb] = s;
    }
    if (tid == 0) a.lampart[pb] = ((sl[0] + sl[1]) + sl[2]) + sl[3];
}

// dlambda[h] = sum of the partials of head h; dL/dw[c] = sum of channel c's partials
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
    const int j = blockIdx.x, tid = threadIdx.x;
    __shared__ float red[256];
    float s = 0.f;
    if (j < a.heads) {
        // partial index = (b * heads + h) * pre_blocks + blk
        for (int k = tid; k < a.batch * a.pre_blocks; k += 256) {
            const int bb = k / a.pre_blocks, blk = k % a.pre_blocks;
            s += a.lampart[((int64_t)bb * a.heads + j) * a.pre_blocks + blk];
        }
    } else {
        const int c = j - a.heads;
        for (int k = tid; k < a.n_part; k += 256) s += a.wpart[(int64_t)c * a.n_part + k];
    }
    red[tid] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) {
        if (j < a.heads) {
            if (a.dlam) a.dlam[j] = red[0];
        } else {
            a.dnorm_w[j - a.heads] = red[0];
        }
    }
}

// ------------------------------------------------------------------------------------------------
// dQ: a block of 4 waves owns 128 queries of one head, 32 per wave, and walks the key tiles.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdArgs a) {
    __shared__ __align__(16) unsigned char smem[kKStages * kKStage];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, h2 = lane >> 5;
    // the last query tiles see the most keys under causal masking: they go first
    const int qt = gridDim.y - 1 - blockIdx.y, h = blockIdx.x % a.heads, b = blockIdx.x / a.heads;
    const int q0 = qt * 128, qw0 = q0 + wave * 32, qrow = qw0 + n;
    const int off = a.seq_k - a.seq_q;
    const bool qok = qrow < a.seq_q;
    const int qr = qok ? qrow : 0;
    const int64_t row = ((int64_t)b * a.heads + h) * a.seq_q + qr;

    // per-lane query operands (B operands, lane = query n): Q1, Q2 (for S^T) and go (for dP^T)
    bf16x8 bq1[4], bq2[4], bg[8];
    {
        const bf16* q1p = (const bf16*)a.q1 + b * a.q1s[0] + (int64_t)qr * a.q1s[1] + (int64_t)h * a.q1s[2] + 8 * h2;
        const bf16* q2p = (const bf16*)a.q2 + b * a.q2s[0] + (int64_t)qr * a.q2s[1] + (int64_t)h * a.q2s[2] + 8 * h2;
        const bf16* gp = a.go + row * kDV + 8 * h2;
        const bf16x8 z = {};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bq1[kk] = qok ? ld_global_bf16x8(q1p + 16 * kk) : z;
            bq2[kk] = qok ? ld_global_bf16x8(q2p + 16 * kk) : z;
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) bg[kk] = qok ? ld_global_bf16x8(gp + 16 * kk) : z;
    }
    const float lse1 = qok ? a.lse[2 * row] : 0.f, lse2 = qok ? a.lse[2 * row + 1] : 0.f;
    const float D1 = qok ? a.dd[2 * row] : 0.f, D2 = qok ? a.dd[2 * row + 1] : 0.f;
    const float lam = a.lam[h];
    const float c = a.scale_log2;

    int nkt = (a.seq_k + kBN - 1) / kBN;
    if (a.causal) nkt = min(nkt, (min(q0 + 127, a.seq_q - 1) + off) / kBN + 1);
    const bool wave_active = qw0 < a.seq_q;
    const int wave_qlast = min(qw0 + 31, a.seq_q - 1);
    // last key each lane's query sees
    const int qlim = a.causal ? min(qrow + off, a.seq_k - 1) : a.seq_k - 1;

    const bf16* k1b = (const bf16*)a.k1 + b * a.k1s[0] + (int64_t)h * a.k1s[2];
    const bf16* k2b = (const bf16*)a.k2 + b * a.k2s[0] + (int64_t)h * a.k2s[2];
    const bf16* vb = (const bf16*)a.v + b * a.vs[0] + (int64_t)h * a.vs[2];

    f32x16 dq1[2], dq2[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) { dq1[mt] = f32x16{}; dq2[mt] = f32x16{}; }

    // key-tile DMA: thread tid fills K1 and K2 slot tid and V slots tid, tid + 256; rows past the
    // last key are fetched from the last one (their weights are masked to zero)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int k_row = slot_row<kD>(tid), k_col = slot_chunk<kD>(tid);
    const int v_row0 = slot_row<kDV>(tid), v_row1 = v_row0 + 16;
    const int v_col0 = slot_chunk<kDV>(tid), v_col1 = slot_chunk<kDV>(tid + 256);
    // the slots' byte offsets within a full tile, computed once; a ragged last tile recomputes them
    // with its rows clamped
    auto slot_offsets = [&](int last, uint32_t* o) __attribute__((always_inline)) {
        o[0] = (uint32_t)(min(k_row, last) * a.k1s[1] + k_col * 8) * 2u;
        o[1] = (uint32_t)(min(k_row, last) * a.k2s[1] + k_col * 8) * 2u;
        o[2] = (uint32_t)(min(v_row0, last) * a.vs[1] + v_col0 * 8) * 2u;
        o[3] = (uint32_t)(min(v_row1, last) * a.vs[1] + v_col1 * 8) * 2u;
    };
    uint32_t full_off[4];
    slot_offsets(kBN - 1, full_off);
    auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
        const int last = min(kBN, a.seq_k - kt * kBN) - 1;
        const uint32_t st = lds0 + stage * kKStage + wave_u * 1024;
        uint32_t o[4] = {full_off[0], full_off[1], full_off[2], full_off[3]};
        if (__builtin_expect(last < kBN - 1, 0)) slot_offsets(last, o);
        dma16(k1b + (int64_t)kt * kBN * a.k1s[1], o[0], st);
        dma16(k2b + (int64_t)kt * kBN * a.k2s[1], o[1], st + kKTile);
        const bf16* vt = vb + (int64_t)kt * kBN * a.vs[1];
        dma16(vt, o[2], st + 2 * kKTile);
        dma16(vt, o[3], st + 2 * kKTile + 4096);
    };

    // one key tile; !full: some (query, key) pair of the wave's 32 x 32 block is not visible
    auto compute = [&](auto ST, bool full, int k0) __attribute__((always_inline)) {
        const unsigned char* K1s = smem + decltype(ST)::value * kKStage;
        const unsigned char* K2s = K1s + kKTile;
        const unsigned char* Vs = K1s + 2 * kKTile;
        // S^T = K Q^T (lane = query n, 16 keys), dP^T = V go^T
        f32x16 s1 = f32x16{}, s2 = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            s1 = mfma32x32x16(lds16(K1s + rowop_b(n, kk, h2)), bq1[kk], s1);
            s2 = mfma32x32x16(lds16(K2s + rowop_b(n, kk, h2)), bq2[kk], s2);
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) dp = mfma32x32x16(lds16(Vs + rowop_v(n, kk, h2)), bg[kk], dp);
        f32x16 p1, p2, ds1, ds2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p1[r] = fast_exp2(fmaf(s1[r], c, -lse1));
            p2[r] = fast_exp2(fmaf(s2[r], c, -lse2));
        }
        if (!full) {
            asm volatile("");   // keeps this a branch: full tiles skip the test
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + (r >> 2) * 8 + h2 * 4 + (r & 3);
                const bool vis = qok && key <= qlim;
                p1[r] = vis ? p1[r] : 0.f;
                p2[r] = vis ? p2[r] : 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            ds1[r] = p1[r] * (dp[r] - D1);
            ds2[r] = p2[r] * (dp[r] - D2);   // the factor -lambda is applied to dQ2 once, at the store
        }
        // dQ_k^T += K_k^T dS_k^T (k index = keys)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 b1 = c_to_b(ds1, kb), b2 = c_to_b(ds2, kb);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                dq1[mt] = mfma32x32x16(tr_pair(K1s, trop_b(lane, kb, mt, 0), trop_b(lane, kb, mt, 1)), b1, dq1[mt]);
                dq2[mt] = mfma32x32x16(tr_pair(K2s, trop_b(lane, kb, mt, 0), trop_b(lane, kb, mt, 1)), b2, dq2[mt]);
            }
        }
    };
    auto tile = [&](auto ST, int kt) __attribute__((always_inline)) {
        const int k0 = kt * kBN;
        if (!wave_active || (a.causal && k0 > wave_qlast + off)) return;
        compute(ST, qw0 + kBN <= a.seq_q && k0 + kBN <= a.seq_k && (!a.causal || k0 + kBN - 1 <= qw0 + off), k0);
    };
    // key tiles in pairs, one block barrier per pair: a ring of four stages holds the pair being
    // worked on and the next pair in flight, unrolled by two pairs so that every LDS address is a
    // register plus a constant
    auto pair = [&](int kt, auto S0, auto S1, auto N0, auto N1) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(kVmcnt[0]);   // this thread's DMA of tiles kt, kt + 1 landed
        __syncthreads();   // both landed everywhere; the stages of the previous pair are free
        if (kt + 2 < nkt) issue(kt + 2, decltype(N0)::value);
        if (kt + 3 < nkt) issue(kt + 3, decltype(N1)::value);
        tile(S0, kt);
        if (kt + 1 < nkt) tile(S1, kt + 1);
    };
    for (int kt = 0; kt < nkt && kt < 2; ++kt) issue(kt, kt);
    // the query operands and the first tiles have landed: from here on the compiler sees no
    // outstanding loads of its own and adds no waits on the key-tile DMA
    __builtin_amdgcn_s_waitcnt(kVmcnt[0]);
    for (int kt = 0; kt < nkt; kt += 4) {
        pair(kt, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        if (kt + 2 < nkt) pair(kt + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
    }
    if (!qok) return;
    // dQ_k = s dS_k K_k; lane (n, h2) holds d = 32 mt + (r / 4) * 8 + 4 h2 + r % 4 of query n
    const float sc2 = -lam * a.scale;   // dS2 was accumulated without its factor -lambda
    bf16* o1p = (bf16*)a.dq1 + b * a.dq1s[0] + (int64_t)qrow * a.dq1s[1] + (int64_t)h * a.dq1s[2];
    bf16* o2p = (bf16*)a.dq2 + b * a.dq2s[0] + (int64_t)qrow * a.dq2s[1] + (int64_t)h * a.dq2s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 x1, x2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x1[j] = (bf16)(dq1[mt][g * 4 + j] * a.scale);
                x2[j] = (bf16)(dq2[mt][g * 4 + j] * sc2);
            }
            *(bf16x4*)(o1p + mt * 32 + g * 8 + h2 * 4) = x1;
            *(bf16x4*)(o2p + mt * 32 + g * 8 + h2 * 4) = x2;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// dK, dV: a block of 4 waves owns 128 keys of one head, 32 per wave, and walks the query tiles.
// Each lane holds its key's K1, K2 and V rows as MFMA B operands; the gradient accumulators
// (dK1^T, dK2^T, dV^T of the wave's 32 keys, 128 registers) sit in AGPRs. One wave per SIMD.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(BwdArgs a) {
    __shared__ __align__(16) unsigned char sq[kQStages * kQStage];
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = tid & 63;
    const int n = lane & 31, h2 = lane >> 5;
    // the first key tiles see the most queries under causal masking: they go first
    const int kt = blockIdx.y, h = blockIdx.x % a.heads, b = blockIdx.x / a.heads;
    const int k0 = kt * 128, kw0 = k0 + wave * 32, key = kw0 + n;
    const int off = a.seq_k - a.seq_q;
    const float lam = a.lam[h];
    const float c = a.scale_log2;
    const bool wave_active = kw0 < a.seq_k;

    // B operands of this lane's key (lane n = key, 16-byte chunk 2 kk + h2); keys past the end
    // read the last key (their weights are masked to zero)
    bf16x8 kr1[4], kr2[4], vr[8];
    {
        const int kr = min(key, a.seq_k - 1);
        const bf16* k1p = (const bf16*)a.k1 + b * a.k1s[0] + (int64_t)kr * a.k1s[1] + (int64_t)h * a.k1s[2] + 8 * h2;
        const bf16* k2p = (const bf16*)a.k2 + b * a.k2s[0] + (int64_t)kr * a.k2s[1] + (int64_t)h * a.k2s[2] + 8 * h2;
        const bf16* vp = (const bf16*)a.v + b * a.vs[0] + (int64_t)kr * a.vs[1] + (int64_t)h * a.vs[2] + 8 * h2;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            kr1[kk] = ld_global_bf16x8(k1p + 16 * kk);
            kr2[kk] = ld_global_bf16x8(k2p + 16 * kk);
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) vr[kk] = ld_global_bf16x8(vp + 16 * kk);
    }

    f32x16 dk1[2], dk2[2], dv[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) { dk1[mt] = f32x16{}; dk2[mt] = f32x16{}; }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) dv[ct] = f32x16{};

    // query tiles that see any of the block's keys
    const int nqt = (a.seq_q + kBN - 1) / kBN;
    const int qt0 = a.causal ? max(0, (k0 - off) / kBN) : 0;
    const bf16* q1b = (const bf16*)a.q1 + b * a.q1s[0] + (int64_t)h * a.q1s[2];
    const bf16* q2b = (const bf16*)a.q2 + b * a.q2s[0] + (int64_t)h * a.q2s[2];
    const int64_t rowb = ((int64_t)b * a.heads + h) * a.seq_q;

    // query-tile DMA: thread tid fills Q1 and Q2 slot tid and go slots tid, tid + 256; waves 1 and
    // 2 also fetch the rows' log-sum-exp and D values (64 floats each). Rows past the last query
    // are fetched from the last one (their weights are masked to zero).
    const uint32_t lds_sq = (uint32_t)(uintptr_t)(lds_u8_t*)sq;
    const int q_row = slot_row<kD>(tid), q_col = slot_chunk<kD>(tid);
    const int g_row0 = slot_row<kDV>(tid), g_row1 = g_row0 + 16;
    const int g_col0 = slot_chunk<kDV>(tid), g_col1 = slot_chunk<kDV>(tid + 256);
    // the slots' byte offsets within a full tile, computed once; a ragged last tile recomputes them
    // with its rows clamped
    auto slot_offsets = [&](int last, uint32_t* o) __attribute__((always_inline)) {
        o[0] = (uint32_t)(min(q_row, last) * a.q1s[1] + q_col * 8) * 2u;
        o[1] = (uint32_t)(min(q_row, last) * a.q2s[1] + q_col * 8) * 2u;
        o[2] = (uint32_t)(min(g_row0, last) * kDV + g_col0 * 8) * 2u;
        o[3] = (uint32_t)(min(g_row1, last) * kDV + g_col1 * 8) * 2u;
    };
    uint32_t full_off[4];
    slot_offsets(kBN - 1, full_off);
    auto issue_q = [&](int qt, int stage) __attribute__((always_inline)) {
        const int i0 = qt * kBN;
        const int last = min(kBN, a.seq_q - i0) - 1;
        const uint32_t st = lds_sq + stage * kQStage + wave * 1024;
        uint32_t o[4] = {full_off[0], full_off[1], full_off[2], full_off[3]};
        if (__builtin_expect(last < kBN - 1, 0)) slot_offsets(last, o);
        dma16(q1b + (int64_t)i0 * a.q1s[1], o[0], st);
        dma16(q2b + (int64_t)i0 * a.q2s[1], o[1], st + kKTile);
        const bf16* gb = a.go + (rowb + i0) * kDV;
        dma16(gb, o[2], st + 2 * kKTile);
        dma16(gb, o[3], st + 2 * kKTile + 4096);
        if (wave == 1 || wave == 2) {
            // lane i fetches float i of the tile's 32 rows x 2 (clamped to the last row): the
            // log-sum-exp by wave 1 and D by wave 2, so that no wave issues more DMA than the rest
            const uint32_t sst = lds_sq + stage * kQStage + kQStats + (wave - 1) * 256;
            const uint32_t fo = (uint32_t)min(lane, 2 * last + 1) * 4u;
            dma4((wave == 1 ? a.lse : a.dd) + 2 * (rowb + i0), fo, sst);
        }
    };

    // S_k = Q_k K_k^T and dP = go V^T of one query tile (rows = queries, lane = key)
    auto scores = [&](const unsigned char* Q1s, f32x16& dp, f32x16& s1, f32x16& s2) __attribute__((always_inline)) {
        const unsigned char* Q2s = Q1s + kKTile;
        const unsigned char* Gs = Q1s + 2 * kKTile;
        dp = f32x16{}; s1 = f32x16{}; s2 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) dp = mfma32x32x16(lds16(Gs + rowop_v(n, kk, h2)), vr[kk], dp);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            s1 = mfma32x32x16(lds16(Q1s + rowop_b(n, kk, h2)), kr1[kk], s1);
            s2 = mfma32x32x16(lds16(Q2s + rowop_b(n, kk, h2)), kr2[kk], s2);
        }
    };
    // weights and score gradients of one tile as bf16 B operands (k index = queries)
    auto weights = [&](const unsigned char* Q1s, bool full, int i0, const f32x16& dp, const f32x16& s1,
                       const f32x16& s2, bf16x8* b1, bf16x8* b2, bf16x8* bp) __attribute__((always_inline)) {
        const float* svl = (const float*)(Q1s + kQStats);   // lse [32][2]
        const float* svd = svl + 64;                          // dd [32][2]
        // register r holds query row 8 (r / 4) + 4 h2 + r % 4
        f32x16 p1, p2, dm1, dm2, ds1, ds2, pc;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            // rows 8g + 4h2 .. +3: their (map 1, map 2) pairs are 8 consecutive floats
            const int q4 = 8 * g + 4 * h2;
            const f32x4 l01 = *(const f32x4*)(svl + 2 * q4), l23 = *(const f32x4*)(svl + 2 * q4 + 4);
            const f32x4 d01 = *(const f32x4*)(svd + 2 * q4), d23 = *(const f32x4*)(svd + 2 * q4 + 4);
            const float lse1[4] = {l01[0], l01[2], l23[0], l23[2]}, lse2[4] = {l01[1], l01[3], l23[1], l23[3]};
            const float dd1[4] = {d01[0], d01[2], d23[0], d23[2]}, dd2[4] = {d01[1], d01[3], d23[1], d23[3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * g + j;
                p1[r] = fast_exp2(fmaf(s1[r], c, -lse1[j]));
                p2[r] = fast_exp2(fmaf(s2[r], c, -lse2[j]));
                dm1[r] = dp[r] - dd1[j];
                dm2[r] = dp[r] - dd2[j];
            }
        }
        if (!full) {
            asm volatile("");   // keeps this a branch: full tiles skip the test
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = i0 + (r >> 2) * 8 + 4 * h2 + (r & 3);
                const bool vis = q < a.seq_q && key < a.seq_k && (!a.causal || key <= q + off);
                p1[r] = vis ? p1[r] : 0.f;
                p2[r] = vis ? p2[r] : 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            ds1[r] = p1[r] * dm1[r];
            ds2[r] = p2[r] * dm2[r];   // the factor -lambda is applied to dK2 once, at the store
            pc[r] = fmaf(-lam, p2[r], p1[r]);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) { b1[kb] = c_to_b(ds1, kb); b2[kb] = c_to_b(ds2, kb); bp[kb] = c_to_b(pc, kb); }
    };
    // dK_k^T += Q_k^T dS_k and dV^T += go^T (A1 - lambda A2) (k index = queries)
    auto grads = [&](const unsigned char* Q1s, const bf16x8* b1, const bf16x8* b2, const bf16x8* bp) __attribute__((always_inline)) {
        const unsigned char* Q2s = Q1s + kKTile;
        const unsigned char* Gs = Q1s + 2 * kKTile;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                mfma_agpr(dk1[mt], tr_pair(Q1s, trop_b(lane, kb, mt, 0), trop_b(lane, kb, mt, 1)), b1[kb]);
                mfma_agpr(dk2[mt], tr_pair(Q2s, trop_b(lane, kb, mt, 0), trop_b(lane, kb, mt, 1)), b2[kb]);
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                mfma_agpr(dv[ct], tr_pair(Gs, trop_v(lane, kb, ct, 0), trop_v(lane, kb, ct, 1)), bp[kb]);
        }
    };
    // one query tile; !full: some (query, key) pair of the wave's 32 x 32 block is not visible
    auto compute = [&](const unsigned char* Q1s, bool full, int i0) __attribute__((always_inline)) {
        f32x16 dp, s1, s2;
        bf16x8 b1[2], b2[2], bp[2];
        scores(Q1s, dp, s1, s2);
        weights(Q1s, full, i0, dp, s1, s2, b1, b2, bp);
        grads(Q1s, b1, b2, bp);
    };
    auto tile_full = [&](int i0) { return i0 + kBN <= a.seq_q && kw0 + kBN <= a.seq_k && (!a.causal || kw0 + kBN - 1 <= i0 + off); };
    auto tile_skip = [&](int i0) { return !wave_active || (a.causal && i0 + kBN - 1 + off < kw0); };
    // two query tiles per block barrier; slots S0, S1 hold them, N0, N1 take the pair after next.
    // FAST: both tiles are unmasked for every wave of the block, and tile B's score MFMAs run
    // beside tile A's vector work, tile A's gradient MFMAs beside tile B's.
    auto pair = [&](auto FAST, int qt, auto S0, auto S1, auto N0, auto N1) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(kVmcnt[0]);   // this thread's DMA of tiles qt, qt + 1 landed
        __syncthreads();   // every thread's loads landed; the slots of the previous pair are free
        if (qt + 2 < nqt) issue_q(qt + 2, decltype(N0)::value);
        if (qt + 3 < nqt) issue_q(qt + 3, decltype(N1)::value);
        const unsigned char* QA = sq + decltype(S0)::value * kQStage;
        const unsigned char* QB = sq + decltype(S1)::value * kQStage;
        const int iA = qt * kBN, iB = iA + kBN;
        if constexpr (decltype(FAST)::value) {
            // 64 MFMAs in a fixed order: tile A's 16 score MFMAs, tile B's 16 (each followed by
            // the vector work of one row of tile A), tile A's 16 gradient MFMAs (each followed by
            // one row of tile B), tile B's 16. Every operand read is issued kLead MFMAs ahead of
            // its use; a scheduling barrier after each step keeps the order.
            constexpr int kLead = 4;
            f32x16 dpA = {}, s1A = {}, s2A = {}, dpB = {}, s1B = {}, s2B = {};
            f32x16 ds1A, ds2A, pcA, ds1B, ds2B, pcB;
            bf16x8 b1A[2], b2A[2], bpA[2], b1B[2], b2B[2], bpB[2];
            bf16x8 op[64];
            f32x4 st[2][4];   // lse and dd of one group of four rows, for tile A then tile B
            auto read_op = [&](int m) __attribute__((always_inline)) {
                const unsigned char* T = (m < 16 || (m >= 32 && m < 48)) ? QA : QB;
                const int i = m & 15;
                if (m < 32) {
                    if (i < 8) op[m] = lds16(T + 2 * kKTile + rowop_v(n, i, h2));
                    else op[m] = lds16(T + (i & 1) * kKTile + rowop_b(n, (i - 8) >> 1, h2));
                } else {
                    const int kb = i >> 3, jj = i & 7;
                    if (jj < 4) op[m] = tr_pair(T + (jj & 1) * kKTile, trop_b(lane, kb, jj >> 1, 0), trop_b(lane, kb, jj >> 1, 1));
                    else op[m] = tr_pair(T + 2 * kKTile, trop_v(lane, kb, jj - 4, 0), trop_v(lane, kb, jj - 4, 1));
                }
            };
            auto issue = [&](int m) __attribute__((always_inline)) {
                const int i = m & 15;
                if (m < 32) {
                    f32x16& dp = m < 16 ? dpA : dpB;
                    f32x16& s1 = m < 16 ? s1A : s1B;
                    f32x16& s2 = m < 16 ? s2A : s2B;
                    if (i < 8) dp = mfma32x32x16(op[m], vr[i], dp);
                    else if (!(i & 1)) s1 = mfma32x32x16(op[m], kr1[(i - 8) >> 1], s1);
                    else s2 = mfma32x32x16(op[m], kr2[(i - 8) >> 1], s2);
                } else {
                    const bf16x8* b1 = m < 48 ? b1A : b1B;
                    const bf16x8* b2 = m < 48 ? b2A : b2B;
                    const bf16x8* bp = m < 48 ? bpA : bpB;
                    const int kb = i >> 3, jj = i & 7;
                    if (jj < 4) {
                        if (jj & 1) mfma_agpr_ready(dk2[jj >> 1], op[m], b2[kb]);
                        else mfma_agpr_ready(dk1[jj >> 1], op[m], b1[kb]);
                    } else {
                        mfma_agpr_ready(dv[jj - 4], op[m], bp[kb]);
                    }
                }
            };
            auto read_stats = [&](const unsigned char* T, int g, f32x4* out) __attribute__((always_inline)) {
                const float* svl = (const float*)(T + kQStats);   // lse [32][2]
                const float* svd = svl + 64;                        // dd [32][2]
                const int q4 = 8 * g + 4 * h2;
                out[0] = *(const f32x4*)(svl + 2 * q4);
                out[1] = *(const f32x4*)(svl + 2 * q4 + 4);
                out[2] = *(const f32x4*)(svd + 2 * q4);
                out[3] = *(const f32x4*)(svd + 2 * q4 + 4);
            };
            // row r (query 8 (r / 4) + 4 h2 + r % 4) of one tile: weights, score gradients
            auto row = [&](int r, const f32x4* sv, const f32x16& dp, const f32x16& s1, const f32x16& s2,
                           f32x16& ds1, f32x16& ds2, f32x16& pc) __attribute__((always_inline)) {
                const int j = r & 3;
                const float lse1 = sv[j >> 1][2 * (j & 1)], lse2 = sv[j >> 1][2 * (j & 1) + 1];
                const float dd1 = sv[2 + (j >> 1)][2 * (j & 1)], dd2 = sv[2 + (j >> 1)][2 * (j & 1) + 1];
                const float p1 = fast_exp2(fmaf(s1[r], c, -lse1));
                const float p2 = fast_exp2(fmaf(s2[r], c, -lse2));
                ds1[r] = p1 * (dp[r] - dd1);
                ds2[r] = p2 * (dp[r] - dd2);   // the factor -lambda is applied to dK2 once, at the store
                pc[r] = fmaf(-lam, p2, p1);
            };
#pragma unroll
            for (int m = 0; m < kLead; ++m) read_op(m);
            read_stats(QA, 0, st[0]);
            __builtin_amdgcn_sched_barrier(0);
            static_for<64>([&](auto M) __attribute__((always_inline)) {
                constexpr int m = decltype(M)::value;
                if (m + kLead < 64) read_op(m + kLead);
                issue(m);
                if (m >= 16 && m < 32) {
                    const int r = m - 16;
                    if ((r & 3) == 0 && r > 0) read_stats(QA, r >> 2, st[0]);
                    row(r, st[0], dpA, s1A, s2A, ds1A, ds2A, pcA);
                    if (r == 15) {
                        read_stats(QB, 0, st[1]);
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) { b1A[kb] = c_to_b(ds1A, kb); b2A[kb] = c_to_b(ds2A, kb); bpA[kb] = c_to_b(pcA, kb); }
                    }
                } else if (m >= 32 && m < 48) {
                    const int r = m - 32;
                    if ((r & 3) == 0 && r > 0) read_stats(QB, r >> 2, st[1]);
                    row(r, st[1], dpB, s1B, s2B, ds1B, ds2B, pcB);
                    if (r == 15) {
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) { b1B[kb] = c_to_b(ds1B, kb); b2B[kb] = c_to_b(ds2B, kb); bpB[kb] = c_to_b(pcB, kb); }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            if (!tile_skip(iA)) compute(QA, tile_full(iA), iA);
            if (qt + 1 < nqt && !tile_skip(iB)) compute(QB, tile_full(iB), iB);
        }
    };
    // Tiles [qs, qm) are unmasked for the whole block and go through the FAST pairs; the others
    // (the causal diagonal, ragged ends) through the masked ones. Both bounds are qt0 plus a
    // multiple of four, so ring slot = (tile - qt0) modulo 4 in every loop, each unrolled by two
    // pairs so that every LDS address is a register plus a constant.
    int qs = nqt, qm = nqt;
    if (k0 + 128 <= a.seq_k) {
        const int qf = a.causal ? max(qt0, (k0 + 127 - off + kBN - 1) / kBN) : qt0;
        const int qe = a.seq_q / kBN;   // tiles below this one hold no row past the end
        const int q4 = qt0 + (qf - qt0 + 3) / 4 * 4;
        if (q4 + 4 <= qe) { qs = q4; qm = q4 + (qe - q4) / 4 * 4; }
    }
    for (int qt = qt0; qt < nqt && qt < qt0 + 2; ++qt) issue_q(qt, qt - qt0);
    // the key operands and the first tiles have landed: from here on the compiler sees no
    // outstanding loads of its own and adds no waits on the query-tile DMA
    __builtin_amdgcn_s_waitcnt(kVmcnt[0]);
    int qt = qt0;
    for (; qt < qs; qt += 4) {
        pair(std::false_type{}, qt, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        if (qt + 2 < nqt) pair(std::false_type{}, qt + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
    }
    for (; qt < qm; qt += 4) {
        pair(std::true_type{}, qt, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        pair(std::true_type{}, qt + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
    }
    for (; qt < nqt; qt += 4) {
        pair(std::false_type{}, qt, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        if (qt + 2 < nqt) pair(std::false_type{}, qt + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
    }
    agpr_drain(dk1[0], dk1[1], dk2[0], dk2[1]);
    agpr_drain(dv[0], dv[1], dv[2], dv[3]);
    if (key >= a.seq_k) return;
    const float sc2 = -lam * a.scale;   // dS2 was accumulated without its factor -lambda
    bf16* k1p = (bf16*)a.dk1 + b * a.dk1s[0] + (int64_t)key * a.dk1s[1] + (int64_t)h * a.dk1s[2];
    bf16* k2p = (bf16*)a.dk2 + b * a.dk2s[0] + (int64_t)key * a.dk2s[1] + (int64_t)h * a.dk2s[2];
    bf16* vp = (bf16*)a.dv + b * a.dvs[0] + (int64_t)key * a.dvs[1] + (int64_t)h * a.dvs[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            bf16x4 x1, x2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x1[j] = (bf16)(dk1[mt][g * 4 + j] * a.scale);
                x2[j] = (bf16)(dk2[mt][g * 4 + j] * sc2);
            }
            *(bf16x4*)(k1p + mt * 32 + g * 8 + h2 * 4) = x1;
            *(bf16x4*)(k2p + mt * 32 + g * 8 + h2 * 4) = x2;
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            bf16x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = (bf16)dv[ct][g * 4 + j];
            *(bf16x4*)(vp + ct * 32 + g * 8 + h2 * 4) = x;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init: gradients of the four vectors, one wave
// per row.
__global__ __launch_bounds__(64) void lambda_bwd_kernel(const float* lq1, const float* lk1, const float* lq2,
                                                        const float* lk2, const float* dlam, int dim, float* dlq1,
                                                        float* dlk1, float* dlq2, float* dlk2) {
    const int r = blockIdx.x, lane = threadIdx.x;
    const int64_t o = (int64_t)r * dim;
    float s1 = 0.f, s2 = 0.f;
    for (int j = lane; j < dim; j += 64) {
        s1 = fmaf(lq1[o + j], lk1[o + j], s1);
        s2 = fmaf(lq2[o + j], lk2[o + j], s2);
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    const float e1 = dlam[r] * expf(s1), e2 = dlam[r] * expf(s2);
    for (int j = lane; j < dim; j += 64) {
        dlq1[o + j] = e1 * lk1[o + j];
        dlk1[o + j] = e1 * lq1[o + j];
        dlq2[o + j] = -e2 * lk2[o + j];
        dlk2[o + j] = -e2 * lq2[o + j];
    }
}

}  // namespace

size_t bwd_workspace_bytes(int batch, int heads, int seq_q) {
    const size_t rows = (size_t)batch * heads * seq_q;
    const size_t n_part = (size_t)batch * heads * ((seq_q + kPreRows - 1) / kPreRows);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    return up(rows * kDV * 2) + up(rows * 2 * sizeof(float)) + up(n_part * kDV * sizeof(float)) +
           up(n_part * sizeof(float));
}

hipError_t launch_bwd(BwdArgs a, void* workspace, hipStream_t stream) {
    const size_t rows = (size_t)a.batch * a.heads * a.seq_q;
    const int pre_blocks = (a.seq_q + kPreRows - 1) / kPreRows;
    a.pre_blocks = pre_blocks;
    a.n_part = a.batch * a.heads * pre_blocks;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    unsigned char* w = (unsigned char*)workspace;
    a.go = (bf16*)w;
    w += up(rows * kDV * 2);
    a.dd = (float*)w;
    w += up(rows * 2 * sizeof(float));
    a.wpart = (float*)w;
    w += up((size_t)a.n_part * kDV * sizeof(float));
    a.lampart = (float*)w;

    hipLaunchKernelGGL(bwd_pre_kernel, dim3(pre_blocks, a.heads, a.batch), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(a.heads * a.batch, (a.seq_q + 127) / 128), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(a.heads * a.batch, (a.seq_k + 127) / 128), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int nred = a.heads + ((a.epi && a.dnorm_w) ? kDV : 0);
    if (a.dlam || a.dnorm_w) {
        hipLaunchKernelGGL(bwd_reduce_kernel, dim3(nred), dim3(256), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_lambda_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                             const float* dlam, int n, int dim, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                             hipStream_t stream) {
    hipLaunchKernelGGL(lambda_bwd_kernel, dim3(n), dim3(64), 0, stream, lq1, lk1, lq2, lk2, dlam, dim, dlq1, dlk1,
                       dlq2, dlk2);
    return hipGetLastError();
}

}  // namespace diffattn
