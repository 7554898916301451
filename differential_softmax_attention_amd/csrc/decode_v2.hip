// DIFF V2 decode: the new token's query heads against a KV cache, bf16, d = 128, on MFMA.
//
// In DIFF V2 the two maps of a pair are two query heads of one GQA group, and every head of the
// group reads the group's single K and V cache ("Differential Transformer: softmax can't say
// zero, so it subtracts", section "DIFF V2: what the authors changed"; "Differential Transformer
// V2": decoding reads the cache as ordinary GQA attention does). Decode is bound by reading the
// cache, so the kernel reads each cached K and V row once for all G = 2h / h_kv query heads of
// the group: the heads are the N dimension of the MFMA tiles.
//
// Split-K: the cache of each (batch, KV head) is cut into n_splits slices; one 64-lane wave
// streams one slice in 32-key tiles through a private 3-stage LDS ring (global_load_lds, no
// block barrier). Per tile, S = Q K^T on v_mfma_f32_32x32x16_bf16 (32 head rows, G of them used,
// x 32 keys, k = 128 in eight steps). The heads are the M dimension so that the 8-row blocks
// holding no head fall on registers the kernel never touches: a lane carries 4 ceil(G/8) scores
// (4 for G <= 8), not 16. Scores are scaled by scale * log2(e) in fp32, base-2 weights are rounded
// to bf16 and staged through a small LDS tile, read back by the transposing LDS read as the A
// operand of O = P V, whose B operand V comes from the same read of the V tile. The slice's
// partial (shift, sum, 128-wide accumulator per head) goes to the workspace; v2_decode_reduce
// merges the slices of each head in split order (log-sum-exp) and forms O_{2p} - lambda_p O_{2p+1}.
// No atomics: the result is bitwise reproducible.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_tile.hpp"

namespace diffattn {

namespace {

constexpr int kBN = 32;                       // keys per tile
constexpr int kD = 128;                       // head width (K, V and output)
constexpr int kKBytes = kBN * kD * 2;
constexpr int kVBytes = kBN * kD * 2;
constexpr int kStageBytes = kKBytes + kVBytes;
constexpr int kStages = 3;
constexpr int kLoadsK = kKBytes / (64 * 16);  // DMA instructions per lane per K tile (8)
constexpr int kLoadsV = kVBytes / (64 * 16);
static_assert(kStages == 3 && kLoadsK + kLoadsV == 16, "the ring's vmcnt waits count 16 loads per tile, 3 stages");
constexpr int kPart = 4 + kD;                 // shift, sum, two pad words, o[128]
constexpr int kMaxGroup = 32;                 // heads per group that fit the MFMA's M = 32
constexpr int kPRow = 72;                     // bytes per key row of the P staging tile: 32 heads + 8 pad
constexpr int kPBytes = kBN * kPRow;
template <int V>
struct StageC { static constexpr int value = V; };
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kMaxLog2 = 64.0f;                   // unshifted weights stay below 2^64
constexpr float kMaxLog2Shifted = 15.0f;            // shifted weights below 2^15
constexpr float kMinSum = 8.673617379884035e-19f;   // 2^-60: a head whose lane sums are all below this has no weight yet
constexpr float kUnshiftedRange = 60.0f;            // first-tile maxima within +-60 (base 2)

// RB = ceil(G / 8): the 8-row blocks of the 32-row MFMA tiles that hold the group's heads
template <int RB>
__global__ __launch_bounds__(64) void v2_decode_split_kernel(V2DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int n = lane & 31;   // column of the 32x32 tiles: the key of S, the channel of O; the head of the Q fragment
    const int h2 = lane >> 5;  // which half of the MFMA k-dimension this lane feeds
    const int G = a.group;

    int len = a.cache_len;
    if (a.cache_lens) len = min(max(a.cache_lens[b], 1), a.cache_len);
    const int ks = split * a.split_len;
    const int ke = min(ks + a.split_len, len);
    const int ntiles = ke > ks ? (ke - ks + kBN - 1) / kBN : 0;

    // ---- Q fragments (A operand of S = Q K^T): lane (n, h2) holds q[head n][16kk + 8h2 .. +7]
    //      as given, zero for rows past the group; the scale is applied to the fp32 scores.
    bf16x8 bq[kD / 16];
    {
        const bool ok = n < G;
        const bf16* qp = (const bf16*)a.q + b * a.qs[0] + (int64_t)(g * G + (ok ? n : 0)) * a.qs[2] + 8 * h2;
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) {
            const bf16x8 z = {};
            bq[kk] = ok ? ld_global_bf16x8(qp + 16 * kk) : z;
        }
    }

    // ---- tile DMA: lane i fills K slots i + 64j and V slots i + 64j (j < 8) of a stage
    // contiguous cache: batch b's rows; paged: the pool (the batch stride is the page stride), a
    // tile of 32 keys starting at a multiple of 32 lying in one page
    const bool paged = a.pc.block_table != nullptr;
    const bf16* kbase = (const bf16*)a.k + (int64_t)g * a.kcs[2];
    const bf16* vbase = (const bf16*)a.v + (int64_t)g * a.vcs[2];
    if (!paged) {
        kbase += b * a.kcs[0] + (int64_t)ks * a.kcs[1];
        vbase += b * a.vcs[0] + (int64_t)ks * a.vcs[1];
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
    // paged: the slice's page indices, 64 at a time, one per lane (lane i holds page slot
    // 64 w + i of the slice), so that a tile's lookup is a lane read rather than a memory load
    // with its latency in front of the tile's DMA
    const int first_slot = paged ? ks / a.pc.page_size : 0;
    const int last_slot = paged ? (ke - 1) / a.pc.page_size : 0;
    int win = -1, pvec = 0;
    // tiles are issued in order, so the next tile's page slot (relative to first_slot) and first
    // row within the page advance by one tile at a time: no division per tile (the page size and
    // the slice start are multiples of the 32-key tile)
    int next_slot = 0, next_in = paged ? ks - first_slot * a.pc.page_size : 0;
    // lane i fills K and V slots i + 64j of a stage (row (i + 64j) / 16, swizzled chunk): byte
    // offsets within a whole tile
    uint32_t koffg[kLoadsK], voffg[kLoadsV];
#pragma unroll
    for (int j = 0; j < kLoadsK; ++j) {
        const int s = lane + 64 * j, row = s >> 4;
        koffg[j] = (uint32_t)(row * a.kcs[1] + ((s & 15) ^ k_swz<kD>(row)) * 8) * 2u;
    }
#pragma unroll
    for (int j = 0; j < kLoadsV; ++j) {
        const int s = lane + 64 * j, row = s >> 4;
        voffg[j] = (uint32_t)(row * a.vcs[1] + v_logical(row, s & 15) * 8) * 2u;
    }
    auto issue_tile = [&](int t, auto stage_c) __attribute__((always_inline)) {
        const uint32_t st = lds0 + decltype(stage_c)::value * kStageBytes;
        const int last = min(kBN, ke - ks - t * kBN) - 1;   // last valid row of this tile
        const bf16 *kb, *vb;
        if (paged) {
            if ((next_slot >> 6) != win) {
                win = next_slot >> 6;
                const int sl = first_slot + win * 64 + lane;
                const int p = sl <= last_slot ? a.pc.block_table[(int64_t)b * a.pc.bt_stride + sl] : 0;
                pvec = min(max(p, 0), a.pc.num_pages - 1);
            }
            const int64_t pg = __builtin_amdgcn_readlane(pvec, next_slot & 63), in = next_in;
            kb = kbase + pg * a.kcs[0] + in * a.kcs[1];
            vb = vbase + pg * a.vcs[0] + in * a.vcs[1];
            next_in += kBN;
            if (next_in == a.pc.page_size) {
                next_in = 0;
                ++next_slot;
            }
        } else {
            kb = kbase + (int64_t)t * kBN * a.kcs[1];
            vb = vbase + (int64_t)t * kBN * a.vcs[1];
        }
        if (last == kBN - 1) {
            // a whole tile: the offsets computed once
#pragma unroll
            for (int j = 0; j < kLoadsK; ++j) dma16(kb, koffg[j], st + j * 1024);
#pragma unroll
            for (int j = 0; j < kLoadsV; ++j) dma16(vb, voffg[j], st + kKBytes + j * 1024);
        } else {
            // the slice's last tile: rows past its end read the last row
#pragma unroll
            for (int j = 0; j < kLoadsK; ++j) {
                const int s = lane + 64 * j;
                const int row = s >> 4;
                const int col = (s & 15) ^ k_swz<kD>(row);
                dma16(kb, (uint32_t)(min(row, last) * a.kcs[1] + col * 8) * 2u, st + j * 1024);
            }
#pragma unroll
            for (int j = 0; j < kLoadsV; ++j) {
                const int s = lane + 64 * j;
                const int row = s >> 4;
                const int col = v_logical(row, s & 15);
                dma16(vb, (uint32_t)(min(row, last) * a.vcs[1] + col * 8) * 2u, st + kKBytes + j * 1024);
            }
        }
    };

    // per-lane LDS offsets of the MFMA operands: K (B operand of S = Q K^T) row n, chunk
    // 2kk + h2; V (B operand of O = P V) through the transposing read, lane (n, h2) receiving
    // channel 32 ct + n of keys 16kb + 4h2 .. +3 and 16kb + 8 + 4h2 .. +3; P (A operand of O) through
    // the same read from the staging tile, lane (n, h2) receiving head n of those keys
    const int koff0 = n * (kD * 2) + ((h2 ^ k_swz<kD>(n)) * 16);
    int voff0, pr_off;
    {
        const int Gq = lane >> 4, L = lane & 15;
        const int row = 4 * (Gq >> 1) + (L >> 2);
        const int c = (Gq & 1) * 2 + ((L >> 1) & 1);
        voff0 = row * (kD * 2) + v_phys(row, c) * 16 + (L & 1) * 8;
        pr_off = row * kPRow + ((Gq & 1) * 16 + 4 * (L & 3)) * 2;
    }
    // P staging tile: [key][head], rows of kPRow bytes; lane (n, h2) writes key n, heads
    // 8rb + 4h2 .. +3 (8 bytes per row block). Zeroed once: heads past 8 RB are never written and
    // feed only output rows that are not stored.
    unsigned char* const ps = smem + kStages * kStageBytes;
    const int pw_off = n * kPRow + 8 * h2;
#pragma unroll
    for (int i = 0; i < kPBytes / 256; ++i) *(uint32_t*)(ps + 4 * (lane + 64 * i)) = 0u;

    // S = Q K^T: lane (n, h2) holds score register 4rb + j = head 8rb + 4h2 + j against key n,
    // and O = P V the same heads against channel 32 ct + n, so each lane carries only the 4 RB
    // registers that can hold heads of the group (the other rows of the 32-row tiles stay unused)
    constexpr int NR = 4 * RB;
    f32x16 o[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o[ct] = f32x16{};
    float m[NR], l[NR];       // per head: shift (equal over the 32 lanes of a half), this lane's sum
#pragma unroll
    for (int r = 0; r < NR; ++r) { m[r] = 0.f; l[r] = 0.f; }
    bool shifted = false;
    // the bf16 pairs {1, 0} and {0, 1} that pick one weight of a packed pair, held in VGPRs: as a
    // constant, {1, 0} is folded into the inline operand 1.0, whose reading by v_dot2c_f32_bf16
    // is not the pair the compiler meant
    uint32_t e_lo_u = 0x00003f80u, e_hi_u = 0x3f800000u;
    asm volatile("" : "+v"(e_lo_u), "+v"(e_hi_u));
    const bf16x2 e_lo = __builtin_bit_cast(bf16x2, e_lo_u), e_hi = __builtin_bit_cast(bf16x2, e_hi_u);
    // maximum over the 32 keys of a tile (the lanes of one half)
    auto half_max = [&](float v) __attribute__((always_inline)) {
#pragma unroll
        for (int msk = 1; msk < 32; msk <<= 1) v = fmax_nc(v, lane_xor(v, (lane ^ msk) << 2));
        return v;
    };

    if (0 < ntiles) issue_tile(0, StageC<0>{});
    if (1 < ntiles) issue_tile(1, StageC<1>{});
    // one tile in stage S (a constant: the loop is unrolled by the three stages, so every LDS
    // address is a register plus an immediate)
    auto tile_step = [&](int t, auto stage_c) __attribute__((always_inline)) {
        constexpr int S = decltype(stage_c)::value;
        // tile t+2 goes into the stage of tile t-1, whose operand reads the previous iteration's
        // MFMAs consumed: issued before the wait, so three tiles are in flight while this wave
        // waits and two while it computes. Loads complete in order, so the wait for tile t leaves
        // the later tiles' 16 loads each in flight.
        if (t + kStages - 1 < ntiles) {
            issue_tile(t + kStages - 1, StageC<(S + kStages - 1) % kStages>{});
            __builtin_amdgcn_s_waitcnt(0x8F70);                   // vmcnt(32)
        } else if (t + 1 < ntiles) {
            __builtin_amdgcn_s_waitcnt(0x4F70);                   // vmcnt(16)
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)
        }
        const unsigned char* st = smem + S * kStageBytes;

        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) s = mfma32x32x16(bq[kk], lds16(st + (koff0 ^ (kk << 5))), s);
        float x[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) x[r] = s[r] * a.scale_log2;   // base-2 units, fp32
        // keys past the slice end were fetched from a clamped address: drop them
        if (ks + (t + 1) * kBN > ke && ks + t * kBN + n >= ke) {
#pragma unroll
            for (int r = 0; r < NR; ++r) x[r] = -INFINITY;
        }
        auto move_shift = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float mx = half_max(x[r]);
                if (!(half_max(l[r]) < kMinSum)) mx = fmax_nc(mx, 0.f);   // a head with weight keeps its scale or raises it
                const float al = fast_exp2(-mx);
                l[r] *= al;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) o[ct][r] *= al;
                x[r] -= mx;
                m[r] += mx;
            }
        };
        if (t == 0) {
            bool out = false;
#pragma unroll
            for (int r = 0; r < NR; ++r) out |= !(fabsf(half_max(x[r])) <= kUnshiftedRange);
            if (__builtin_amdgcn_ballot_w64(out)) {
                move_shift();
                shifted = true;
            }
        } else if (shifted) {
#pragma unroll
            for (int r = 0; r < NR; ++r) x[r] -= m[r];
        }
        // a weight above the mode's bound moves the shifts first (exact: the shift travels with
        // the partial)
        float xm = x[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) xm = fmax_nc(xm, x[r]);
        if (__builtin_amdgcn_ballot_w64(!(xm <= (shifted ? kMaxLog2Shifted : kMaxLog2)))) {
            shifted = true;
            move_shift();
        }
        // weights rounded to bf16, their sums taken from the same bf16 values, staged as P
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            bf16x2 w2[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 4 * rb + 2 * i;
                w2[i] = bf16x2{(bf16)fast_exp2(x[r]), (bf16)fast_exp2(x[r + 1])};
                l[r] = __builtin_amdgcn_fdot2_f32_bf16(w2[i], e_lo, l[r], false);
                l[r + 1] = __builtin_amdgcn_fdot2_f32_bf16(w2[i], e_hi, l[r + 1], false);
            }
            *(u32x2*)(ps + pw_off + 16 * rb) = u32x2{__builtin_bit_cast(uint32_t, w2[0]), __builtin_bit_cast(uint32_t, w2[1])};
        }
        // O += P V over the tile's two 16-key halves
        const unsigned char* Vs = st + kKBytes;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const i16x4 plo = lds_read_tr16((const bf16*)(ps + pr_off + kb * 16 * kPRow));
            const i16x4 phi = lds_read_tr16((const bf16*)(ps + pr_off + (kb * 16 + 8) * kPRow));
            const bf16x8 pa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(plo, phi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const bf16* vp = (const bf16*)(Vs + (voff0 ^ (ct << 6)) + kb * 16 * (kD * 2));
                const i16x4 lo = lds_read_tr16(vp);
                const i16x4 hi = lds_read_tr16(vp + 8 * kD);
                const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[ct] = mfma32x32x16(pa, vb, o[ct]);
            }
        }
    };
    for (int t = 0; t < ntiles; t += kStages) {
        tile_step(t, StageC<0>{});
        if (t + 1 < ntiles) tile_step(t + 1, StageC<1>{});
        if (t + 2 < ntiles) tile_step(t + 2, StageC<2>{});
    }

    // ---- partial of this slice for each head of the group (an empty slice has no weight)
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int msk = 1; msk < 32; msk <<= 1) l[r] += lane_xor(l[r], (lane ^ msk) << 2);
        const int head = 8 * (r >> 2) + 4 * h2 + (r & 3);
        if (head < G) {
            float* w = a.ws + ((((int64_t)b * a.h_kv + g) * a.n_splits + split) * G + head) * kPart;
            if (n == 0) {
                w[0] = ntiles > 0 ? m[r] : -INFINITY;
                w[1] = l[r];
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) w[4 + ct * 32 + n] = o[ct][r];
        }
    }
}

// One block of 128 threads (one per channel) per (pair, batch): merge each head's slices in split
// order, then O_{2p} - lambda O_{2p+1}.
__global__ __launch_bounds__(128) void v2_decode_reduce_kernel(V2DecodeArgs a) {
    const int p = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    const int G = a.group;
    // the two heads of pair p, merged over the splits in split order in one pass (running maximum,
    // sum and channel value rescaled when the maximum rises), so that the loads of eight splits of
    // both heads are in flight together
    const float* w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int j = 2 * p + k;   // query head
        w[k] = a.ws + (((int64_t)b * a.h_kv + j / G) * a.n_splits * G + (j % G)) * kPart;
    }
    const int64_t stride = (int64_t)G * kPart;   // next split of the same head
    float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.f, 0.f}, O[2] = {0.f, 0.f};
#pragma unroll 8
    for (int s = 0; s < a.n_splits; ++s) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float* ws = w[k] + s * stride;
            const float ms = ws[0], ls = ws[1], os = ws[4 + c];
            // an empty slice stored shift -inf, sum 0 and zeros: it changes nothing (selected, not
            // branched, so the loads stay ahead; before the first non-empty slice both shifts are
            // -inf and their difference NaN, which the selects discard)
            const bool empty = ms == -INFINITY;
            const float mn = fmaxf(M[k], ms);
            const float fo = empty ? 1.f : fast_exp2(M[k] - mn), fs = empty ? 0.f : fast_exp2(ms - mn);
            L[k] = fmaf(ls, fs, L[k] * fo);
            O[k] = fmaf(os, fs, O[k] * fo);
            M[k] = empty ? M[k] : mn;
        }
    }
    const float lam = a.lam_sigmoid ? sigmoid_f32(a.lam[(int64_t)b * a.lam_bs + p]) : a.lam[(int64_t)b * a.lam_bs + p];
    float x;
    {
#pragma clang fp contract(off)
        x = O[0] / L[0] - lam * (O[1] / L[1]);
    }
    bf16* op = (bf16*)a.out + b * a.os[0] + (int64_t)p * a.os[2];
    op[c] = (bf16)x;
}

}  // namespace

// Blocks of the split kernel resident at once on the current device (three per CU: the LDS
// ring), cached per device and row-block count.
static int v2_decode_capacity(int rb) {
    static std::atomic<int> cache[64][5];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int c = cache[dev][rb].load(std::memory_order_relaxed);
    if (c > 0) return c;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const size_t lds = (size_t)kStages * kStageBytes + kPBytes;
    hipError_t e = hipErrorInvalidValue;
    switch (rb) {
        case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, v2_decode_split_kernel<1>, 64, lds); break;
        case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, v2_decode_split_kernel<2>, 64, lds); break;
        case 3: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, v2_decode_split_kernel<3>, 64, lds); break;
        default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, v2_decode_split_kernel<4>, 64, lds); break;
    }
    if (e != hipSuccess || per_cu <= 0) per_cu = 3;
    c = cus * per_cu;
    cache[dev][rb].store(c, std::memory_order_relaxed);
    return c;
}

// Slices per (batch, KV head). A block ends with its partial's stores, and its slot takes about
// one loaded memory round trip (a few tiles' time) to free, so short slices cost; too few blocks
// leave resident slots idle in the last round. The count minimises rounds x (tiles per slice +
// kSplitOverheadTiles), with at least 8 tiles per slice.
constexpr int kSplitOverheadTiles = 4;

int v2_decode_num_splits(int batch, int h_kv, int group, int cache_len) {
    const int64_t units = (int64_t)batch * h_kv;
    const int64_t cap = v2_decode_capacity((group + 7) / 8);
    const int max_splits = std::max(1, std::min((cache_len + 255) / 256, 4096));
    const int64_t tiles = (cache_len + kBN - 1) / kBN;
    int best = 1;
    int64_t best_cost = -1;
    for (int sp = 1; sp <= max_splits; ++sp) {
        const int64_t rounds = (units * sp + cap - 1) / cap;
        const int64_t cost = rounds * ((tiles + sp - 1) / sp + kSplitOverheadTiles);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = sp;
        }
    }
    int split_len = (cache_len + best - 1) / best;
    split_len = (split_len + kBN - 1) / kBN * kBN;
    return (cache_len + split_len - 1) / split_len;
}

static int v2_decode_split_len(int cache_len, int splits) {
    int split_len = (cache_len + splits - 1) / splits;
    return (split_len + kBN - 1) / kBN * kBN;
}

size_t v2_decode_workspace_bytes(int batch, int h, int h_kv, int cache_len) {
    const int G = 2 * h / h_kv;
    return (size_t)batch * h_kv * v2_decode_num_splits(batch, h_kv, G, cache_len) * G * kPart * sizeof(float);
}

bool v2_decode_group_ok(int group) { return group >= 2 && group <= kMaxGroup; }

hipError_t launch_v2_decode(V2DecodeArgs a, hipStream_t stream) {
    a.n_splits = v2_decode_num_splits(a.batch, a.h_kv, a.group, a.cache_len);
    a.split_len = v2_decode_split_len(a.cache_len, a.n_splits);
    const dim3 grid(a.n_splits, a.h_kv, a.batch);
    const size_t lds = (size_t)kStages * kStageBytes + kPBytes;
    switch ((a.group + 7) / 8) {
        case 1: hipLaunchKernelGGL(v2_decode_split_kernel<1>, grid, dim3(64), lds, stream, a); break;
        case 2: hipLaunchKernelGGL(v2_decode_split_kernel<2>, grid, dim3(64), lds, stream, a); break;
        case 3: hipLaunchKernelGGL(v2_decode_split_kernel<3>, grid, dim3(64), lds, stream, a); break;
        case 4: hipLaunchKernelGGL(v2_decode_split_kernel<4>, grid, dim3(64), lds, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(v2_decode_reduce_kernel, dim3(a.h, a.batch), dim3(kD), 0, stream, a);
    return hipGetLastError();
}

}  // namespace diffattn
