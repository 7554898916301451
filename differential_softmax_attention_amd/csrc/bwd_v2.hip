// DIFF V2 backward on bf16 MFMA (gfx950): d = 128, query heads 2p and 2p+1 of one GQA group form
// pair p and read their group's K and V; lambda per (token, pair), given or as the sigmoid of its
// logit; no norm ("softmax can't say zero, so it subtracts", section "DIFF V2: what the authors
// changed"; "Differential Transformer V2").
//
// Gradients of out_p = A_{2p} V - lambda A_{2p+1} V for L = sum(dout * out), by the chain rule:
//   go = dout_p,  dP = go V^T (shared by both heads),  D_k = go . (A_k V) per row,
//   dS_{2p} = A_{2p} (dP - D_1),  dS_{2p+1} = -lambda A_{2p+1} (dP - D_2),
//   dQ_j = s dS_j K,  dK = s sum over the group's heads of dS_j^T Q_j,
//   dV = sum over the group's pairs of (A_{2p} - lambda A_{2p+1})^T go_p,
//   dlambda = -go . (A_{2p+1} V) per row (times sigmoid'(z) = lambda (1 - lambda) for logits).
// The training forward supplies each head's log-sum-exp and A_k V.
//
// Kernels (no atomics; every sum in a fixed order):
//  - bwd_v2_pre: half a wave per (row, pair): go (a copy of dout, head-major for the DMA), D_1, D_2,
//    lambda after the sigmoid, and dlambda.
//  - bwd_v2_dq: 32 queries of one pair per wave, walking key tiles (K and V of the group through
//    a four-slot LDS ring, two tiles per block barrier); each K row fragment feeds both heads'
//    scores and each transposed K fragment both heads' dQ. Pairs of unmasked tiles run their 80
//    MFMAs in a fixed order, the second tile's score MFMAs beside the first tile's vector work.
//  - bwd_v2_dkdv: 32 keys of one KV head per wave (K and V rows in registers), walking the query
//    tiles of every pair of the group; dK gathers both heads of every pair, dV every pair. Items
//    (query tile, pair) come two per block barrier; where neither holds a masked (query, key) pair
//    for any wave of the block, their 96 MFMAs run in a fixed order with the second item's score
//    MFMAs beside the first item's vector work and the first item's gradient MFMAs beside the
//    second's, each operand read issued four MFMAs ahead.
// The dQ and dK/dV accumulators sit in AGPRs (inline-asm MFMAs); tiles are 128 wide in the
// backward layout of bwd_tile.hpp.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_tile.hpp"
#include "bwd_tile.hpp"

namespace diffattn {

namespace {

using namespace bwdt;
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kTile = kBN * kD * 2;          // bytes of one 32-row, 128-wide tile
constexpr int kPreRows = 64;                 // rows per pre block (4 waves x 16 rows)
// dQ key-tile stage: K | V
constexpr int kKStage = 2 * kTile;
// dK/dV LDS by operand type, four ring slots per region: Q_{2p} | Q_{2p+1} | go_p | statistics
// (lse [32][2], dd [32][2], lambda [32]); every slot offset fits the LDS immediate
constexpr int kQRing = 4;
constexpr int kQ2Off = kQRing * kTile;
constexpr int kGOff = 2 * kQRing * kTile;
constexpr int kStOff = 3 * kQRing * kTile;
constexpr int kStSlot = 3 * 256;
constexpr int kDkdvLds = kStOff + kQRing * kStSlot;

// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_v2_pre_kernel(V2BwdArgs a) {
    const int blk = blockIdx.x, p = blockIdx.y, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // a wave takes its rows two at a time: lanes 0-31 one row, lanes 32-63 the next, each lane
    // the four channels c0 .. c0 + 3 (16-byte map loads, 8-byte dout loads and go stores)
    const int hl = lane >> 5, c0 = 4 * (lane & 31);
    // steps of two rows in chunks of two steps: a chunk's loads are issued while the previous
    // chunk is reduced (rows past the end read row 0 and are not used)
    constexpr int R = kPreRows / 4, CH = 2, NC = R / (2 * CH);
    struct Chunk { f32x4 a1[CH], a2[CH]; bf16x4 dy[CH]; };
    auto row_of = [&](int c, int k) { return blk * kPreRows + wave * R + 2 * (c * CH + k) + hl; };
    auto load_chunk = [&](int c, Chunk& r) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int i = row_of(c, k);
            const int ii = i < a.seq ? i : 0;
            const float* mp = a.maps + (((int64_t)b * a.seq + ii) * a.h + p) * 2 * kD;   // token-major
            r.a1[k] = *(const f32x4*)(mp + c0);
            r.a2[k] = *(const f32x4*)(mp + kD + c0);
            const bf16* dyp = (const bf16*)a.dout + b * a.dos[0] + (int64_t)ii * a.dos[1] + (int64_t)p * a.dos[2];
            r.dy[k] = *(const bf16x4*)(dyp + c0);
        }
    };
    auto reduce_chunk = [&](int c, const Chunk& r) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int i = row_of(c, k);
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = (float)r.dy[k][j];
            // the half-wave sums run on every lane; only valid rows are stored
            const float D1 = half_sum((y[0] * r.a1[k][0] + y[1] * r.a1[k][1]) + (y[2] * r.a1[k][2] + y[3] * r.a1[k][3]));
            const float D2 = half_sum((y[0] * r.a2[k][0] + y[1] * r.a2[k][1]) + (y[2] * r.a2[k][2] + y[3] * r.a2[k][3]));
            if (i >= a.seq) continue;
            const int64_t row = ((int64_t)b * a.h + p) * a.seq + i;      // head-major row
            const int64_t tok = ((int64_t)b * a.seq + i) * a.h + p;      // token-major (lam, maps)
            *(bf16x4*)(a.go + row * kD + c0) = r.dy[k];
            if ((lane & 31) == 0) {
                const float z = a.lam[tok];
                const float lam = a.lam_sigmoid ? sigmoid_f32(z) : z;
                const float dl = -D2;
                a.dlam[tok] = a.lam_sigmoid ? dl * lam * (1.f - lam) : dl;
                a.lamr[row] = lam;
                *(float2*)(a.dd + 2 * row) = make_float2(D1, D2);
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
}

// ------------------------------------------------------------------------------------------------
// dQ: a block of 4 waves owns 128 queries of one pair, 32 per wave, and walks the key tiles.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_v2_dq_kernel(V2BwdArgs a) {
    __shared__ __align__(16) unsigned char smem[4 * kKStage];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, h2 = lane >> 5;
    // the last query tiles see the most keys under causal masking: they go first. Within a query
    // tile, (batch, KV head) varies fastest: blocks are dealt round-robin over the 8 XCDs in order
    // of linear block index, so when h_kv * batch is a multiple of 8 the pairs of one (batch, KV
    // head) run on one XCD and share its L2 copy of their K and V tiles.
    const int units = a.h_kv * a.batch, unit = blockIdx.x % units;
    const int g = unit % a.h_kv, b = unit / a.h_kv, p = g * (a.group / 2) + blockIdx.x / units;
    const int qt = gridDim.y - 1 - blockIdx.y;
    const int q0 = qt * 128, qw0 = q0 + wave * 32, qrow = qw0 + n;
    const bool qok = qrow < a.seq;
    const int qr = qok ? qrow : 0;
    const int64_t row = ((int64_t)b * a.h + p) * a.seq + qr;

    // per-lane query operands (B operands, lane = query n): both heads' Q (for S^T) and go (for dP^T)
    bf16x8 bq1[8], bq2[8], bg[8];
    {
        const bf16* q1p = (const bf16*)a.q + b * a.qs[0] + (int64_t)qr * a.qs[1] + (int64_t)(2 * p) * a.qs[2] + 8 * h2;
        const bf16* q2p = q1p + a.qs[2];
        const bf16* gp = a.go + row * kD + 8 * h2;
        const bf16x8 z = {};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            bq1[kk] = qok ? ld_global_bf16x8(q1p + 16 * kk) : z;
            bq2[kk] = qok ? ld_global_bf16x8(q2p + 16 * kk) : z;
            bg[kk] = qok ? ld_global_bf16x8(gp + 16 * kk) : z;
        }
    }
    const float lse1 = qok ? a.lse[2 * row] : 0.f, lse2 = qok ? a.lse[2 * row + 1] : 0.f;
    const float D1 = qok ? a.dd[2 * row] : 0.f, D2 = qok ? a.dd[2 * row + 1] : 0.f;
    const float nlam = qok ? -a.lamr[row] : 0.f;
    const float c = a.scale_log2;

    int nkt = (a.seq + kBN - 1) / kBN;
    if (a.causal) nkt = min(nkt, min(q0 + 127, a.seq - 1) / kBN + 1);
    const bool wave_active = qw0 < a.seq;
    const int wave_qlast = min(qw0 + 31, a.seq - 1);
    const int qlim = a.causal ? qrow : a.seq - 1;   // last key this lane's query sees

    const bf16* kb0 = (const bf16*)a.k + b * a.ks[0] + (int64_t)g * a.ks[2];
    const bf16* vb0 = (const bf16*)a.v + b * a.vs[0] + (int64_t)g * a.vs[2];

    f32x16 dq1[4], dq2[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) { dq1[mt] = f32x16{}; dq2[mt] = f32x16{}; }

    // key-tile DMA: thread tid fills K and V slots tid and tid + 256; rows past the last key are
    // fetched from the last one (their weights are masked to zero)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int r0 = slot_row<kD>(tid), r1 = r0 + 16;
    const int c0 = slot_chunk<kD>(tid), c1 = slot_chunk<kD>(tid + 256);
    // the slots' byte offsets within a full tile, computed once; a ragged last tile recomputes them
    // with its rows clamped
    auto slot_offsets = [&](int last, uint32_t* o) __attribute__((always_inline)) {
        o[0] = (uint32_t)(min(r0, last) * a.ks[1] + c0 * 8) * 2u;
        o[1] = (uint32_t)(min(r1, last) * a.ks[1] + c1 * 8) * 2u;
        o[2] = (uint32_t)(min(r0, last) * a.vs[1] + c0 * 8) * 2u;
        o[3] = (uint32_t)(min(r1, last) * a.vs[1] + c1 * 8) * 2u;
    };
    uint32_t full_off[4];
    slot_offsets(kBN - 1, full_off);
    auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
        const int last = min(kBN, a.seq - kt * kBN) - 1;
        const uint32_t st = lds0 + stage * kKStage + wave_u * 1024;
        const bf16* kt_p = kb0 + (int64_t)kt * kBN * a.ks[1];
        const bf16* vt_p = vb0 + (int64_t)kt * kBN * a.vs[1];
        uint32_t o[4] = {full_off[0], full_off[1], full_off[2], full_off[3]};
        if (__builtin_expect(last < kBN - 1, 0)) slot_offsets(last, o);
        dma16(kt_p, o[0], st);
        dma16(kt_p, o[1], st + 4096);
        dma16(vt_p, o[2], st + kTile);
        dma16(vt_p, o[3], st + kTile + 4096);
    };

    auto compute = [&](int slot, bool full, int k0) __attribute__((always_inline)) {
        const unsigned char* Ks = smem + slot * kKStage;
        const unsigned char* Vs = Ks + kTile;
        // S_j^T = K Q_j^T (lane = query n, 16 keys), dP^T = V go^T
        f32x16 s1 = f32x16{}, s2 = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 kf = lds16(Ks + rowop<kD>(n, kk, h2));
            s1 = mfma32x32x16(kf, bq1[kk], s1);
            s2 = mfma32x32x16(kf, bq2[kk], s2);
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) dp = mfma32x32x16(lds16(Vs + rowop<kD>(n, kk, h2)), bg[kk], dp);
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
            ds2[r] = p2[r] * (dp[r] - D2);   // the row's factor -lambda is applied to dQ_{2p+1} at the store
        }
        // dQ_j^T += K^T dS_j^T (k index = keys); one transposed K fragment serves both heads
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 b1 = c_to_b(ds1, kb), b2 = c_to_b(ds2, kb);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 kt_f = tr_pair(Ks, trop<kD>(lane, kb, mt, 0), trop<kD>(lane, kb, mt, 1));
                mfma_agpr(dq1[mt], kt_f, b1);
                mfma_agpr(dq2[mt], kt_f, b2);
            }
        }
    };
    auto tile_full = [&](int k0) { return qw0 + kBN <= a.seq && k0 + kBN <= a.seq && (!a.causal || k0 + kBN - 1 <= qw0); };
    auto tile_skip = [&](int k0) { return !wave_active || (a.causal && k0 > wave_qlast); };
    // two key tiles per block barrier; slots S0, S1 hold them, N0, N1 take the pair after next.
    // FAST: both tiles are unmasked for every wave of the block; their 80 MFMAs run in a fixed
    // order: tile A's 24 score and dP MFMAs, tile B's 24 beside tile A's rows, tile A's 16 dQ
    // MFMAs beside tile B's rows, tile B's 16, operand reads issued about four MFMAs ahead and a
    // scheduling barrier after each MFMA.
    auto pair = [&](auto FAST, int kt, auto S0, auto S1, auto N0, auto N1) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(kVmcnt[0]);   // this thread's DMA of tiles kt, kt + 1 landed
        __syncthreads();   // every thread's loads landed; the slots of the previous pair are free
        if (kt + 2 < nkt) issue(kt + 2, decltype(N0)::value);
        if (kt + 3 < nkt) issue(kt + 3, decltype(N1)::value);
        const unsigned char* KA = smem + decltype(S0)::value * kKStage;
        const unsigned char* KB = smem + decltype(S1)::value * kKStage;
        if constexpr (decltype(FAST)::value) {
            constexpr int kLead = 4;
            f32x16 s1A = {}, s2A = {}, dpA = {}, s1B = {}, s2B = {}, dpB = {};
            float ds1A[16], ds2A[16], ds1B[16], ds2B[16];
            bf16x8 b1A[2], b2A[2], b1B[2], b2B[2];
            bf16x8 op[48];
            // operands: [0,8) K rows of A, [8,16) V rows of A, [16,32) the same of B, [32,40)
            // transposed K of A, [40,48) of B
            auto opidx = [](int m) constexpr {
                return m < 16 ? (m >> 1) : m < 24 ? 8 + (m - 16) : m < 40 ? 16 + ((m - 24) >> 1)
                     : m < 48 ? 24 + (m - 40) : m < 64 ? 32 + ((m - 48) >> 1) : 40 + ((m - 64) >> 1);
            };
            auto read_op = [&](int o) __attribute__((always_inline)) {
                const unsigned char* T = (o < 16 || (o >= 32 && o < 40)) ? KA : KB;
                if (o < 32) {
                    const int u = o & 15;
                    op[o] = u < 8 ? lds16(T + rowop<kD>(n, u, h2)) : lds16(T + kTile + rowop<kD>(n, u - 8, h2));
                } else {
                    const int u = o & 7, kb = u >> 2, mt = u & 3;
                    op[o] = tr_pair(T, trop<kD>(lane, kb, mt, 0), trop<kD>(lane, kb, mt, 1));
                }
            };
            auto issue_mfma = [&](int m) __attribute__((always_inline)) {
                const bf16x8 o = op[opidx(m)];
                if (m < 48) {
                    const int i = m < 24 ? m : m - 24;
                    f32x16& s1 = m < 24 ? s1A : s1B;
                    f32x16& s2 = m < 24 ? s2A : s2B;
                    f32x16& dp = m < 24 ? dpA : dpB;
                    if (i < 16) {
                        if (i & 1) s2 = mfma32x32x16(o, bq2[i >> 1], s2);
                        else s1 = mfma32x32x16(o, bq1[i >> 1], s1);
                    } else {
                        dp = mfma32x32x16(o, bg[i - 16], dp);
                    }
                } else {
                    const int i = m < 64 ? m - 48 : m - 64, kb = i >> 3, mt = (i >> 1) & 3;
                    if (i & 1) mfma_agpr_ready(dq2[mt], o, m < 64 ? b2A[kb] : b2B[kb]);
                    else mfma_agpr_ready(dq1[mt], o, m < 64 ? b1A[kb] : b1B[kb]);
                }
            };
            // row r of a tile (its 16 registers hold keys k0 + 8 (r / 4) + 4 h2 + r % 4)
            auto row = [&](const f32x16& s1, const f32x16& s2, const f32x16& dp, int r, float* ds1, float* ds2) __attribute__((always_inline)) {
                const float p1 = fast_exp2(fmaf(s1[r], c, -lse1));
                const float p2 = fast_exp2(fmaf(s2[r], c, -lse2));
                ds1[r] = p1 * (dp[r] - D1);
                ds2[r] = p2 * (dp[r] - D2);   // the row's factor -lambda is applied to dQ_{2p+1} at the store
            };
            auto pack = [&](const float* ds1, const float* ds2, int kb, bf16x8* b1, bf16x8* b2) __attribute__((always_inline)) {
                for (int t = 0; t < 8; ++t) { b1[kb][t] = (bf16)ds1[8 * kb + t]; b2[kb][t] = (bf16)ds2[8 * kb + t]; }
            };
            static_for<48>([&](auto O) __attribute__((always_inline)) {
                constexpr int o = decltype(O)::value;
                if (o <= opidx(kLead)) read_op(o);
            });
            __builtin_amdgcn_sched_barrier(0);
            static_for<80>([&](auto M) __attribute__((always_inline)) {
                constexpr int m = decltype(M)::value;
                if (m + kLead < 80) {
                    static_for<48>([&](auto O) __attribute__((always_inline)) {
                        constexpr int o = decltype(O)::value;
                        if (o > opidx(m + kLead - 1) && o <= opidx(m + kLead)) read_op(o);
                    });
                }
                issue_mfma(m);
                if (m >= 24 && m < 48) {
                    const int u = m - 24;   // rows of A: row j after MFMA 24 + floor(3 j / 2)
                    if (u % 3 != 2) {
                        const int r = (2 * u + 2) / 3;
                        row(s1A, s2A, dpA, r, ds1A, ds2A);
                        if ((r & 7) == 7) pack(ds1A, ds2A, r >> 3, b1A, b2A);
                    }
                } else if (m >= 48 && m < 64) {
                    const int r = m - 48;   // rows of B, one after each of A's dQ MFMAs
                    row(s1B, s2B, dpB, r, ds1B, ds2B);
                    if ((r & 7) == 7) pack(ds1B, ds2B, r >> 3, b1B, b2B);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            const int kA = kt * kBN, kB = kA + kBN;
            if (!tile_skip(kA)) compute(decltype(S0)::value, tile_full(kA), kA);
            if (kt + 1 < nkt && !tile_skip(kB)) compute(decltype(S1)::value, tile_full(kB), kB);
        }
    };
    // Key tiles [0, kf) are unmasked for every wave of the block (the causal diagonal and a ragged
    // end come last); the fast pairs take them in whole ring periods of four tiles, so ring slot =
    // tile modulo 4 in both loops, each unrolled by two pairs so that every LDS address is a
    // register plus a constant.
    int kf = 0;
    if (q0 + 128 <= a.seq) kf = (a.causal ? q0 : a.seq) / kBN / 4 * 4;
    for (int kt = 0; kt < nkt && kt < 2; ++kt) issue(kt, kt);
    // the query operands and the first tiles have landed: from here on the compiler sees no
    // outstanding loads of its own and adds no waits on the key-tile DMA
    __builtin_amdgcn_s_waitcnt(kVmcnt[0]);
    int kt = 0;
    for (; kt < kf; kt += 4) {
        pair(std::true_type{}, kt, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        pair(std::true_type{}, kt + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
    }
    for (; kt < nkt; kt += 4) {
        pair(std::false_type{}, kt, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        if (kt + 2 < nkt) pair(std::false_type{}, kt + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
    }
    agpr_drain(dq1[0], dq1[1], dq1[2], dq1[3]);
    agpr_drain(dq2[0], dq2[1], dq2[2], dq2[3]);
    if (!qok) return;
    // dQ_j = s dS_j K; lane (n, h2) holds d = 32 mt + (r / 4) * 8 + 4 h2 + r % 4 of query n
    const float sc2 = nlam * a.scale;   // dS_{2p+1} was accumulated without the row's factor -lambda
    bf16* o1p = (bf16*)a.dq + b * a.dqs[0] + (int64_t)qrow * a.dqs[1] + (int64_t)(2 * p) * a.dqs[2];
    bf16* o2p = o1p + a.dqs[2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            bf16x4 x1, x2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x1[j] = (bf16)(dq1[mt][gq * 4 + j] * a.scale);
                x2[j] = (bf16)(dq2[mt][gq * 4 + j] * sc2);
            }
            *(bf16x4*)(o1p + mt * 32 + gq * 8 + h2 * 4) = x1;
            *(bf16x4*)(o2p + mt * 32 + gq * 8 + h2 * 4) = x2;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// dK, dV of one key tile: the block's 4 waves own 128 keys of KV head g, 32 per wave, and walk the
// query tiles of every pair of the group, from the last tile down (down) or from the first tile the
// keys see up. Each lane holds its key's K and V rows as MFMA B operands; dK^T and dV^T of the
// wave's 32 keys (128 registers) sit in AGPRs. One wave per SIMD. Ends with the LDS ring still in
// use by other waves: a second call needs a block barrier first.
__device__ __attribute__((always_inline)) inline void dkdv_key_tile(const V2BwdArgs& a, unsigned char* sq, int kt,
                                                                    int g, int b, bool down) {
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = tid & 63;
    const int n = lane & 31, h2 = lane >> 5;
    const int k0 = kt * 128, kw0 = k0 + wave * 32, key = kw0 + n;
    const int npair = a.group / 2;        // pairs of this KV group: g * npair .. + npair - 1
    const float c = a.scale_log2;
    const bool wave_active = kw0 < a.seq;

    // B operands of this lane's key (lane n = key, 16-byte chunk 2 kk + h2); keys past the end
    // read the last key (their weights are masked to zero)
    bf16x8 kr[8], vr[8];
    {
        const int kr_ = min(key, a.seq - 1);
        const bf16* kp = (const bf16*)a.k + b * a.ks[0] + (int64_t)kr_ * a.ks[1] + (int64_t)g * a.ks[2] + 8 * h2;
        const bf16* vp = (const bf16*)a.v + b * a.vs[0] + (int64_t)kr_ * a.vs[1] + (int64_t)g * a.vs[2] + 8 * h2;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            kr[kk] = ld_global_bf16x8(kp + 16 * kk);
            vr[kk] = ld_global_bf16x8(vp + 16 * kk);
        }
    }

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) { dk[t] = f32x16{}; dv[t] = f32x16{}; }

    // work items: (query tile, pair of the group), query tile outermost; item it reads query tile
    // qbase + qstep * (it / npair)
    const int nqt = (a.seq + kBN - 1) / kBN;
    const int qt0 = a.causal ? k0 / kBN : 0;
    const int nit = (nqt - qt0) * npair;
    const int qbase = down ? nqt - 1 : qt0, qstep = down ? -1 : 1;

    // stage DMA: thread tid fills Q_{2p}, Q_{2p+1} and go_p slots tid and tid + 256; waves 1, 2 and
    // 3 also fetch the rows' log-sum-exp and D (64 floats each) and lambda (32 floats), one each.
    // Rows past the last query are fetched from the last one (their weights are masked to zero).
    const uint32_t lds_sq = (uint32_t)(uintptr_t)(lds_u8_t*)sq;
    const int r0 = slot_row<kD>(tid), r1 = r0 + 16;
    const int c0 = slot_chunk<kD>(tid), c1 = slot_chunk<kD>(tid + 256);
    // the slots' byte offsets within a full tile, computed once; a ragged last tile recomputes them
    // with its rows clamped (Q_{2p} and Q_{2p+1} share theirs)
    auto slot_offsets = [&](int last, uint32_t* o) __attribute__((always_inline)) {
        o[0] = (uint32_t)(min(r0, last) * a.qs[1] + c0 * 8) * 2u;
        o[1] = (uint32_t)(min(r1, last) * a.qs[1] + c1 * 8) * 2u;
        o[2] = (uint32_t)(min(r0, last) * kD + c0 * 8) * 2u;
        o[3] = (uint32_t)(min(r1, last) * kD + c1 * 8) * 2u;
    };
    uint32_t full_off[4];
    slot_offsets(kBN - 1, full_off);
    auto issue = [&](int it, int stage) __attribute__((always_inline)) {
        const int qt = qbase + qstep * (it / npair), p = g * npair + it % npair;
        const int i0 = qt * kBN;
        const int last = min(kBN, a.seq - i0) - 1;
        const uint32_t st = lds_sq + stage * kTile + wave * 1024;
        const bf16* q1b = (const bf16*)a.q + b * a.qs[0] + (int64_t)i0 * a.qs[1] + (int64_t)(2 * p) * a.qs[2];
        const bf16* q2b = q1b + a.qs[2];
        const int64_t rowb = ((int64_t)b * a.h + p) * a.seq + i0;
        const bf16* gb = a.go + rowb * kD;
        uint32_t o[4] = {full_off[0], full_off[1], full_off[2], full_off[3]};
        if (__builtin_expect(last < kBN - 1, 0)) slot_offsets(last, o);
        dma16(q1b, o[0], st);
        dma16(q1b, o[1], st + 4096);
        dma16(q2b, o[0], st + kQ2Off);
        dma16(q2b, o[1], st + kQ2Off + 4096);
        dma16(gb, o[2], st + kGOff);
        dma16(gb, o[3], st + kGOff + 4096);
        if (wave != 0) {   // one statistics DMA each for waves 1, 2 and 3
            const uint32_t sst = lds_sq + kStOff + stage * kStSlot + (wave - 1) * 256;
            if (wave == 3) {
                dma4(a.lamr + rowb, (uint32_t)min(lane, last) * 4u, sst);
            } else {
                const uint32_t fo = (uint32_t)min(lane, 2 * last + 1) * 4u;
                dma4((wave == 1 ? a.lse : a.dd) + 2 * rowb, fo, sst);
            }
        }
    };

    // Lane offsets of the LDS reads: the go tiles' carry their region base, hidden from the
    // compiler so that it keeps one register per offset and puts only the slot offset into the
    // instruction's immediate; Q_{2p} and Q_{2p+1} share theirs.
    auto opaque = [](int x) __attribute__((always_inline)) { asm("" : "+v"(x)); return x; };
    int ro[8], gro[8], tro[2][4][2], gtro[2][4][2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) { ro[kk] = rowop<kD>(n, kk, h2); gro[kk] = opaque(kGOff + ro[kk]); }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                tro[kb][mt][hi] = trop<kD>(lane, kb, mt, hi);
                gtro[kb][mt][hi] = opaque(kGOff + tro[kb][mt][hi]);
            }
    const int sto = opaque(kStOff + 32 * h2);   // lse of rows 4 h2 + 8 g + 0..3 at + 64 g, dd at + 256
    const int stm = opaque(kStOff + 512 + 16 * h2);   // lambda of the same rows at + 32 g
    // operand of S / dP MFMA i (0-7: go rows for dP, 8-23: Q_{2p} and Q_{2p+1} rows alternately)
    auto rd_s = [&](int slot, int i) __attribute__((always_inline)) -> bf16x8 {
        if (i < 8) return lds16(sq + slot * kTile + gro[i]);
        return lds16(sq + ((i & 1) ? kQ2Off : 0) + slot * kTile + ro[(i - 8) >> 1]);
    };
    // operand of gradient MFMA i (kb = i / 12; i % 12: dK mt 0 from Q_{2p}, from Q_{2p+1}, mt 1 ...,
    // then dV ct 0-3)
    auto rd_g = [&](int slot, int i) __attribute__((always_inline)) -> bf16x8 {
        const int kb = i / 12, jj = i % 12;
        if (jj < 8) return tr_pair(sq + ((jj & 1) ? kQ2Off : 0) + slot * kTile, tro[kb][jj >> 1][0], tro[kb][jj >> 1][1]);
        return tr_pair(sq + slot * kTile, gtro[kb][jj - 8][0], gtro[kb][jj - 8][1]);
    };
    auto mfma_s = [&](int i, bf16x8 o, f32x16& dp, f32x16& s1, f32x16& s2) __attribute__((always_inline)) {
        if (i < 8) dp = mfma32x32x16(o, vr[i], dp);
        else if (!(i & 1)) s1 = mfma32x32x16(o, kr[(i - 8) >> 1], s1);
        else s2 = mfma32x32x16(o, kr[(i - 8) >> 1], s2);
    };
    // READY: the fixed-order pair loop, whose operands were packed many instructions earlier
    auto mfma_g = [&](int i, bf16x8 o, bf16x8 b1, bf16x8 b2, bf16x8 bp, auto READY) __attribute__((always_inline)) {
        const int jj = i % 12;
        if constexpr (decltype(READY)::value) {
            if (jj < 8) mfma_agpr_ready(dk[jj >> 1], o, (jj & 1) ? b2 : b1);
            else mfma_agpr_ready(dv[jj - 8], o, bp);
        } else {
            if (jj < 8) mfma_agpr(dk[jj >> 1], o, (jj & 1) ? b2 : b1);
            else mfma_agpr(dv[jj - 8], o, bp);
        }
    };
    // statistics of register row r (query 8 (r / 4) + 4 h2 + r % 4) of a slot's tile
    auto st_lse = [&](int slot, int r) __attribute__((always_inline)) {
        return *(const f32x2*)(sq + sto + slot * kStSlot + 64 * (r >> 2) + 8 * (r & 3));
    };
    auto st_dd = [&](int slot, int r) __attribute__((always_inline)) {
        return *(const f32x2*)(sq + sto + slot * kStSlot + 256 + 64 * (r >> 2) + 8 * (r & 3));
    };
    auto st_lam = [&](int slot, int r) __attribute__((always_inline)) {
        return *(const float*)(sq + stm + slot * kStSlot + 32 * (r >> 2) + 4 * (r & 3));
    };
    // one row: weights and score gradients (the factor -lambda inside dS_{2p+1}: the dK sum runs
    // over rows with different lambda)
    auto row_math = [&](float dp, float s1, float s2, f32x2 l, f32x2 d, float lm, float& ds1, float& ds2, float& pc) __attribute__((always_inline)) {
        const float p1 = fast_exp2(fmaf(s1, c, -l[0]));
        const float p2 = fast_exp2(fmaf(s2, c, -l[1]));
        const float nl = -lm;
        ds1 = p1 * (dp - d[0]);
        ds2 = nl * p2 * (dp - d[1]);
        pc = fmaf(nl, p2, p1);
    };
    // one item on its own; !full: some (query, key) pair of the wave's 32 x 32 block is not visible
    auto compute = [&](int slot, bool full, int i0) __attribute__((always_inline)) {
        f32x16 dp = {}, s1 = {}, s2 = {};
#pragma unroll
        for (int i = 0; i < 24; ++i) mfma_s(i, rd_s(slot, i), dp, s1, s2);
        float p1[16], p2[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const f32x2 l = st_lse(slot, r);
            p1[r] = fast_exp2(fmaf(s1[r], c, -l[0]));
            p2[r] = fast_exp2(fmaf(s2[r], c, -l[1]));
        }
        if (!full) {
            asm volatile("");   // keeps this a branch: full tiles skip the test
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = i0 + (r >> 2) * 8 + 4 * h2 + (r & 3);
                const bool vis = q < a.seq && key < a.seq && (!a.causal || key <= q);
                p1[r] = vis ? p1[r] : 0.f;
                p2[r] = vis ? p2[r] : 0.f;
            }
        }
        bf16x8 b1[2], b2[2], bp[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const f32x2 d = st_dd(slot, r);
            const float nl = -st_lam(slot, r);
            b1[r >> 3][r & 7] = (bf16)(p1[r] * (dp[r] - d[0]));
            b2[r >> 3][r & 7] = (bf16)(nl * p2[r] * (dp[r] - d[1]));
            bp[r >> 3][r & 7] = (bf16)fmaf(nl, p2[r], p1[r]);
        }
#pragma unroll
        for (int i = 0; i < 24; ++i) mfma_g(i, rd_g(slot, i), b1[i / 12], b2[i / 12], bp[i / 12], std::false_type{});
    };
    auto item_i0 = [&](int it) { return (qbase + qstep * (it / npair)) * kBN; };
    auto item_full = [&](int i0) { return i0 + kBN <= a.seq && kw0 + kBN <= a.seq && (!a.causal || kw0 + kBN - 1 <= i0); };
    auto item_skip = [&](int i0) { return !wave_active || (a.causal && i0 + kBN - 1 < kw0); };
    // two items per block barrier; slots S0, S1 hold them, N0, N1 take the pair after next.
    // FAST: both items are unmasked for every wave of the block; their 96 MFMAs run in a fixed
    // order: item A's 24 score MFMAs, item B's 24 beside item A's rows, item A's 24 gradient
    // MFMAs beside item B's rows, item B's 24, every operand read four MFMAs ahead and a
    // scheduling barrier after each MFMA.
    auto pair = [&](auto FAST, int it, auto S0, auto S1, auto N0, auto N1) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(kVmcnt[0]);   // this thread's DMA of items it, it + 1 landed
        __syncthreads();   // every thread's loads landed; the slots of the previous pair are free
        if (it + 2 < nit) issue(it + 2, decltype(N0)::value);
        if (it + 3 < nit) issue(it + 3, decltype(N1)::value);
        constexpr int sa = decltype(S0)::value, sb = decltype(S1)::value;
        if constexpr (decltype(FAST)::value) {
            constexpr int kLead = 4;
            f32x16 dpA = {}, s1A = {}, s2A = {}, dpB = {}, s1B = {}, s2B = {};
            float ds1A[16], ds2A[16], pcA[16], ds1B[16], ds2B[16], pcB[16];
            bf16x8 b1A[2], b2A[2], bpA[2], b1B[2], b2B[2], bpB[2];
            bf16x8 op[96];
            // statistics of row group g (rows 4 g .. 4 g + 3 of tile A for g < 4, of B after): lse
            // and D as (map 1, map 2) pairs, two rows per 16-byte read, and lambda of the four rows
            f32x4 gl[8][2], gd[8][2], gm[8];
            // MFMA m: [0,24) scores of A, [24,48) scores of B, [48,72) gradients of A, [72,96) of B
            auto read_op = [&](int m) __attribute__((always_inline)) {
                if (m < 24) op[m] = rd_s(sa, m);
                else if (m < 48) op[m] = rd_s(sb, m - 24);
                else if (m < 72) op[m] = rd_g(sa, m - 48);
                else op[m] = rd_g(sb, m - 72);
            };
            auto issue_mfma = [&](int m) __attribute__((always_inline)) {
                if (m < 24) mfma_s(m, op[m], dpA, s1A, s2A);
                else if (m < 48) mfma_s(m - 24, op[m], dpB, s1B, s2B);
                else if (m < 72) { const int kb = (m - 48) / 12; mfma_g(m - 48, op[m], b1A[kb], b2A[kb], bpA[kb], std::true_type{}); }
                else { const int kb = (m - 72) / 12; mfma_g(m - 72, op[m], b1B[kb], b2B[kb], bpB[kb], std::true_type{}); }
            };
            // row job j: [0,16) rows of A (beside B's scores), [16,32) rows of B (beside A's
            // gradients); job j follows MFMA 24 + (3 j) / 2; its statistics are read two jobs ahead
            auto read_group = [&](int g) __attribute__((always_inline)) {
                const int slot = g < 4 ? sa : sb, rg = g & 3;
                const unsigned char* pl = sq + sto + slot * kStSlot + 64 * rg;
                gl[g][0] = *(const f32x4*)pl;
                gl[g][1] = *(const f32x4*)(pl + 16);
                gd[g][0] = *(const f32x4*)(pl + 256);
                gd[g][1] = *(const f32x4*)(pl + 256 + 16);
                gm[g] = *(const f32x4*)(sq + stm + slot * kStSlot + 32 * rg);
            };
            auto job = [&](int j) __attribute__((always_inline)) {
                const int r = j & 15, g = j >> 2, w = j & 3;
                const f32x2 lj = {gl[g][w >> 1][2 * (w & 1)], gl[g][w >> 1][2 * (w & 1) + 1]};
                const f32x2 dj = {gd[g][w >> 1][2 * (w & 1)], gd[g][w >> 1][2 * (w & 1) + 1]};
                const float mj = gm[g][w];
                if (j < 16) {
                    row_math(dpA[r], s1A[r], s2A[r], lj, dj, mj, ds1A[r], ds2A[r], pcA[r]);
                    if ((r & 7) == 7) {
                        const int kb = r >> 3;
                        for (int t = 0; t < 8; ++t) {
                            b1A[kb][t] = (bf16)ds1A[8 * kb + t]; b2A[kb][t] = (bf16)ds2A[8 * kb + t]; bpA[kb][t] = (bf16)pcA[8 * kb + t];
                        }
                    }
                } else {
                    row_math(dpB[r], s1B[r], s2B[r], lj, dj, mj, ds1B[r], ds2B[r], pcB[r]);
                    if ((r & 7) == 7) {
                        const int kb = r >> 3;
                        for (int t = 0; t < 8; ++t) {
                            b1B[kb][t] = (bf16)ds1B[8 * kb + t]; b2B[kb][t] = (bf16)ds2B[8 * kb + t]; bpB[kb][t] = (bf16)pcB[8 * kb + t];
                        }
                    }
                }
            };
            static_for<kLead>([&](auto M) __attribute__((always_inline)) { read_op(decltype(M)::value); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<96>([&](auto M) __attribute__((always_inline)) {
                constexpr int m = decltype(M)::value;
                if (m + kLead < 96) read_op(m + kLead);
                issue_mfma(m);
                // jobs after MFMA 24 + floor(3 j / 2): j = 0 at 24, 1 at 25, 2 at 27, 3 at 28, ...
                if (m == 20) read_group(0);
                if (m >= 24 && m < 72) {
                    const int u = m - 24;   // u = floor(3 j / 2) has a solution j iff u % 3 != 2
                    if (u % 3 != 2) {
                        const int j = (2 * u + 2) / 3;
                        if ((j & 3) == 0 && (j >> 2) + 1 < 8) read_group((j >> 2) + 1);
                        job(j);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            const int iA = item_i0(it);
            if (!item_skip(iA)) compute(sa, item_full(iA), iA);
            if (it + 1 < nit) {
                const int iB = item_i0(it + 1);
                if (!item_skip(iB)) compute(sb, item_full(iB), iB);
            }
        }
    };
    // Items [is, ie) are unmasked for the whole block and go through the FAST pairs, the others
    // through the masked ones. Both bounds are multiples of four, so ring slot = item modulo 4 in
    // every loop, each unrolled by two pairs so that every LDS address is a register plus a
    // constant.
    int is = nit, ie = nit;
    if (k0 + 128 <= a.seq) {
        const int qf = a.causal ? (k0 + 127 + kBN - 1) / kBN : 0;   // first tile unmasked for all waves
        const int qe = a.seq / kBN;                                    // tiles below hold no row past the end
        // the unmasked tiles [max(qf, qt0), qe) as a range of items in the walk's order
        const int i_f = (down ? nqt - qe : max(qf, qt0) - qt0) * npair;
        const int i_e = (down ? nqt - max(qf, qt0) : qe - qt0) * npair;
        const int i4 = (i_f + 3) / 4 * 4;
        if (i4 + 4 <= i_e) { is = i4; ie = i4 + (i_e - i4) / 4 * 4; }
    }
    for (int it = 0; it < nit && it < 2; ++it) issue(it, it);
    // the key operands and the first tiles have landed: from here on the compiler sees no
    // outstanding loads of its own and adds no waits on the query-tile DMA
    __builtin_amdgcn_s_waitcnt(kVmcnt[0]);
    int it = 0;
    auto fence = [&]() __attribute__((always_inline)) { agpr_fence(dk[0], dk[1], dk[2], dk[3], dv[0], dv[1], dv[2], dv[3]); };
    for (; it < is; it += 4) {
        pair(std::false_type{}, it, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        if (it + 2 < nit) pair(std::false_type{}, it + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
        fence();
    }
    for (; it < ie; it += 4) {
        pair(std::true_type{}, it, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        pair(std::true_type{}, it + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
        fence();
    }
    for (; it < nit; it += 4) {
        pair(std::false_type{}, it, IC<0>{}, IC<1>{}, IC<2>{}, IC<3>{});
        if (it + 2 < nit) pair(std::false_type{}, it + 2, IC<2>{}, IC<3>{}, IC<0>{}, IC<1>{});
        fence();
    }
    agpr_drain(dk[0], dk[1], dk[2], dk[3]);
    agpr_drain(dv[0], dv[1], dv[2], dv[3]);
    if (key >= a.seq) return;
    bf16* kp = (bf16*)a.dk + b * a.dks[0] + (int64_t)key * a.dks[1] + (int64_t)g * a.dks[2];
    bf16* vp = (bf16*)a.dv + b * a.dvs[0] + (int64_t)key * a.dvs[1] + (int64_t)g * a.dvs[2];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x4 xk, xv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xk[j] = (bf16)(dk[t][gq * 4 + j] * a.scale);
                xv[j] = (bf16)dv[t][gq * 4 + j];
            }
            *(bf16x4*)(kp + t * 32 + gq * 8 + h2 * 4) = xk;
            *(bf16x4*)(vp + t * 32 + gq * 8 + h2 * 4) = xv;
        }
    }
}

// Block y of KV head g owns key tiles y and nkt - 1 - y, one after the other. Under causal
// masking the pair sees a fixed number of query tiles (nqt + 4) whatever y is, so every block does
// the same work. The first tile is walked from the last query tile down, the second from its first
// query tile up: blocks that start together then read the same query tile at the same time (each
// block's second walk is at tile t - 4 after t tiles of work). Blocks are dealt round-robin over
// the 8 XCDs in order of linear block index, so when h_kv * batch is a multiple of 8 all blocks of
// one (batch, KV head) run on one XCD, whose L2 then serves a query tile to all of them from one
// fetch instead of each block fetching it again. The loop is kept rolled: one copy of the body.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_v2_dkdv_kernel(V2BwdArgs a) {
    __shared__ __align__(16) unsigned char sq[kDkdvLds];
    const int g = blockIdx.x % a.h_kv, b = blockIdx.x / a.h_kv, y = blockIdx.y;
    const int nkt = (a.seq + 127) / 128;
#pragma clang loop unroll(disable)
    for (int s = 0; s < 2; ++s) {
        const int kt = s ? nkt - 1 - y : y;
        if (s) {
            if (kt <= y) break;   // an odd tile count leaves the middle tile unpaired
            __syncthreads();      // every wave is done with the LDS ring of the first tile
        }
        dkdv_key_tile(a, sq, kt, g, b, s == 0);
    }
}

}  // namespace

size_t v2_bwd_workspace_bytes(int batch, int h, int seq) {
    const size_t rows = (size_t)batch * h * seq;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    return up(rows * kD * 2) + up(rows * 2 * sizeof(float)) + up(rows * sizeof(float));
}

hipError_t launch_v2_bwd(V2BwdArgs a, void* workspace, hipStream_t stream) {
    const size_t rows = (size_t)a.batch * a.h * a.seq;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    unsigned char* w = (unsigned char*)workspace;
    a.go = (bf16*)w;
    w += up(rows * kD * 2);
    a.dd = (float*)w;
    w += up(rows * 2 * sizeof(float));
    a.lamr = (float*)w;

    hipLaunchKernelGGL(bwd_v2_pre_kernel, dim3((a.seq + kPreRows - 1) / kPreRows, a.h, a.batch), dim3(256), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_v2_dq_kernel, dim3(a.h * a.batch, (a.seq + 127) / 128), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_v2_dkdv_kernel, dim3(a.h_kv * a.batch, ((a.seq + 127) / 128 + 1) / 2), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace diffattn
