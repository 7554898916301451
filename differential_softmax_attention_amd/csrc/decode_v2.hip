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
// block barrier). Per tile, S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 head columns,
// G of them used, k = 128 in eight steps), scaled by scale * log2(e) in fp32, base-2 weights, and
// O^T += V^T P^T with V^T read by the transposing LDS read. The slice's partial (shift, sum, 128-wide accumulator per head) goes to
// the workspace; v2_decode_reduce merges the slices of each head in split order (log-sum-exp)
// and forms O_{2p} - lambda_p O_{2p+1}. No atomics: the result is bitwise reproducible.
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
constexpr int kPart = 4 + kD;                 // shift, sum, two pad words, o[128]
constexpr int kMaxGroup = 32;                 // heads per group that fit the MFMA's N = 32

constexpr float kMaxSum = 18446744073709551616.0f;  // 2^64: bound on a lane's 16 weights, unshifted
constexpr float kMaxSumShifted = 32768.0f;          // 2^15: the same bound in shifted mode
constexpr float kMinSum = 8.673617379884035e-19f;   // 2^-60: a column below this has no weight yet
constexpr float kUnshiftedRange = 60.0f;            // first-tile maxima within +-60 (base 2)

__global__ __launch_bounds__(64) void v2_decode_split_kernel(V2DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int n = lane & 31;   // head column within the group
    const int h2 = lane >> 5;  // which half of the MFMA k-dimension this lane feeds
    const int G = a.group;

    int len = a.cache_len;
    if (a.cache_lens) len = min(max(a.cache_lens[b], 1), a.cache_len);
    const int ks = split * a.split_len;
    const int ke = min(ks + a.split_len, len);
    const int ntiles = ke > ks ? (ke - ks + kBN - 1) / kBN : 0;

    // ---- Q fragments (B operand of S^T = K Q^T): lane (n, h2) holds q[head n][16kk + 8h2 .. +7]
    //      as given, zero for columns past the group; the scale is applied to the fp32 scores.
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
    auto issue_tile = [&](int t) __attribute__((always_inline)) {
        const uint32_t st = lds0 + (t % kStages) * kStageBytes;
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
    };

    // per-lane LDS offsets of the MFMA operands (see the prefill kernels)
    const int koff0 = n * (kD * 2) + ((h2 ^ k_swz<kD>(n)) * 16);
    int voff0;
    {
        const int Gq = lane >> 4, L = lane & 15;
        const int row = 4 * (Gq >> 1) + (L >> 2);
        const int c = (Gq & 1) * 2 + ((L >> 1) & 1);
        voff0 = row * (kD * 2) + v_phys(row, c) * 16 + (L & 1) * 8;
    }

    f32x16 o[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o[ct] = f32x16{};
    float m = 0.f, l = 0.f;   // shift and this lane's running sum (column n)
    bool shifted = false;
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    for (int t = 0; t < kStages - 1 && t < ntiles; ++t) issue_tile(t);
    for (int t = 0; t < ntiles; ++t) {
        // loads complete in order: tile t+1's loads may stay in flight
        if (t + 1 < ntiles) __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
        if (t + kStages - 1 < ntiles) issue_tile(t + kStages - 1);  // into the stage of tile t-1
        const unsigned char* st = smem + (t % kStages) * kStageBytes;

        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) s = mfma32x32x16(lds16(st + (koff0 ^ (kk << 5))), bq[kk], s);
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] *= a.scale_log2;   // scores in base-2 units, fp32
        if (ks + (t + 1) * kBN > ke) {
            // rows past the slice end were fetched from a clamped address: drop their keys
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (ks + t * kBN + (r >> 2) * 8 + h2 * 4 + (r & 3) >= ke) s[r] = -INFINITY;
        }
        auto move_shift = [&]() __attribute__((always_inline)) {
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmax_nc(mx, s[r]);
            mx = max_halves(mx);
            if (!(sum_halves(l) < kMinSum)) mx = fmax_nc(mx, 0.f);
            const float al = fast_exp2(-mx);
            l *= al;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) o[ct] *= al;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] -= mx;
            m += mx;
        };
        if (t == 0) {
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmax_nc(mx, s[r]);
            if (__builtin_amdgcn_ballot_w64(!(fabsf(mx) <= kUnshiftedRange))) {
                move_shift();
                shifted = true;
            }
        } else if (shifted) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] -= m;
        }
        bf16x8 p[2];
        float ls;
        auto weights = [&]() __attribute__((always_inline)) {
            float acc = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                bf16x2 pp[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = kb * 8 + 2 * j;
                    pp[j] = bf16x2{(bf16)fast_exp2(s[r]), (bf16)fast_exp2(s[r + 1])};
                    acc = __builtin_amdgcn_fdot2_f32_bf16(pp[j], ones, acc, false);
                }
                p[kb] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                                __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
            }
            ls = acc;
        };
        weights();
        if (__builtin_amdgcn_ballot_w64(!(ls <= (shifted ? kMaxSumShifted : kMaxSum)))) {
            shifted = true;
            move_shift();
            weights();
        }
        l += ls;
        const unsigned char* Vs = st + kKBytes;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const bf16* vp = (const bf16*)(Vs + (voff0 ^ (ct << 6)) + kb * 16 * (kD * 2));
                const i16x4 lo = lds_read_tr16(vp);
                const i16x4 hi = lds_read_tr16(vp + 8 * kD);
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[ct] = mfma32x32x16(va, p[kb], o[ct]);
            }
        }
    }

    // ---- partial of this slice for each head of the group (an empty slice has no weight)
    l = sum_halves(l);
    if (n < G) {
        float* w = a.ws + ((((int64_t)b * a.h_kv + g) * a.n_splits + split) * G + n) * kPart;
        if (h2 == 0) {
            w[0] = ntiles > 0 ? m : -INFINITY;
            w[1] = l;
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) w[4 + ct * 32 + (r >> 2) * 8 + h2 * 4 + (r & 3)] = o[ct][r];
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

int v2_decode_num_splits(int batch, int h_kv, int cache_len) {
    const int units = batch * h_kv;
    const int max_splits = (cache_len + 255) / 256;   // at least 256 keys (8 tiles) per slice
    int splits = (8192 + units - 1) / units;
    splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
    int split_len = (cache_len + splits - 1) / splits;
    split_len = (split_len + kBN - 1) / kBN * kBN;
    return (cache_len + split_len - 1) / split_len;
}

static int v2_decode_split_len(int cache_len, int splits) {
    int split_len = (cache_len + splits - 1) / splits;
    return (split_len + kBN - 1) / kBN * kBN;
}

size_t v2_decode_workspace_bytes(int batch, int h, int h_kv, int cache_len) {
    const int G = 2 * h / h_kv;
    return (size_t)batch * h_kv * v2_decode_num_splits(batch, h_kv, cache_len) * G * kPart * sizeof(float);
}

bool v2_decode_group_ok(int group) { return group >= 2 && group <= kMaxGroup; }

hipError_t launch_v2_decode(V2DecodeArgs a, hipStream_t stream) {
    a.n_splits = v2_decode_num_splits(a.batch, a.h_kv, a.cache_len);
    a.split_len = v2_decode_split_len(a.cache_len, a.n_splits);
    hipLaunchKernelGGL(v2_decode_split_kernel, dim3(a.n_splits, a.h_kv, a.batch), dim3(64),
                       (size_t)kStages * kStageBytes, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(v2_decode_reduce_kernel, dim3(a.h, a.batch), dim3(kD), 0, stream, a);
    return hipGetLastError();
}

}  // namespace diffattn
