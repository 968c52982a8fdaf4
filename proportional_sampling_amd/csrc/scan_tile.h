// scan_tile.h -- the tile machinery shared by the CDF scan and the fused PER
// update: tile loads, weights, the tile-local scan, the fixed-association
// lookback and the monotone tile values.
//
// The CDF of the pages is one serial prefix sum ("trainer: parallel
// build_cdf scan + tiled ... mingru backward", "1. Parallel build_cdf").
// Here it is formed tile by tile (256 threads x 4R elements).  In fp mode
// the result is made exactly monotone and its tile boundaries are made
// consistent, at the cost of changes of a few ulps at most:
//   * tile j's exclusive prefix excl_j = F_g + P_j, where P_j is a DPP tree
//     over the sums of the earlier tiles of its group (non-decreasing in j)
//     and F_g = ((GT_0 + GT_1) + ...) + GT_{g-1} is a serial fold of the
//     group totals, so excl is non-decreasing across group boundaries too;
//   * inside a tile, a running max removes rounding dips between threads;
//   * every tile but the last is clamped from above by excl_{j+1} (which it
//     computes exactly as tile j+1 will) and its last element is set to
//     excl_{j+1}.  So C[end_j - 1] == excl_{j+1} <= C[end_j], the CDF is
//     non-decreasing everywhere, and tile j owns exactly the thresholds in
//     (excl_j, excl_{j+1}] (tile 0 from -inf, the last tile up to +inf).
// Integer mode is exact and needs none of this.
#pragma once

#include <type_traits>

#include "psamp_device.h"

namespace psamp {

constexpr int kScanThreads = 256;
constexpr int kScanGroup = 64;         // tiles per lookback group
constexpr int kWsHeaderWords = 32;     // 256-byte header
constexpr int kSlotWords = 8;          // per tile: {A, GT, MIN} x 2 parities + 2 spare
constexpr int kMinTile = kScanThreads * 4;
constexpr int kSpinLimit = 1 << 21;    // bounded waits (about a second)
constexpr int kGtWords = 4;            // group totals per lane per round trip

enum : int { kSlotA = 0, kSlotGT = 2, kSlotMin = 4 };
enum : int { kHdrCalls = 0, kHdrHw = 1, kHdrErr = 2, kHdrT = 4 };

template <class In> struct ScanAcc;
template <> struct ScanAcc<float> { using type = double; };
template <> struct ScanAcc<uint32_t> { using type = uint64_t; };

__device__ __forceinline__ double to_weight(float p, double alpha, const MathLds* M) {
    return pow_prio(p, alpha, M);
}
__device__ __forceinline__ uint64_t to_weight(uint32_t q, double, const MathLds*) {
    return (uint64_t)q;
}

__device__ __forceinline__ uint64_t* slot_word(uint64_t* slots, uint64_t tile, int kind, int par) {
    return &slots[kSlotWords * tile + kind + par];
}

template <int R, class In>
__device__ __forceinline__ void load_tile(const In* __restrict__ in, int64_t n, int64_t base,
                                          bool vec_ok, In (&v)[R][4]) {
    constexpr int ROW = kScanThreads * 4;
    const int tid = threadIdx.x;
    if (vec_ok && base + (int64_t)R * ROW <= n) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint4 x = *reinterpret_cast<const uint4*>(in + base + r * ROW + 4 * tid);
            v[r][0] = __builtin_bit_cast(In, x.x);
            v[r][1] = __builtin_bit_cast(In, x.y);
            v[r][2] = __builtin_bit_cast(In, x.z);
            v[r][3] = __builtin_bit_cast(In, x.w);
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t i = base + r * ROW + 4 * tid + c;
                v[r][c] = i < n ? in[i] : In(0);
            }
    }
}

// Zero the other parity's status words (A, GT, MIN of every slot below the
// high-water mark, and its T word) so that the next call finds them clean.
__device__ __forceinline__ void clear_other_parity(uint64_t* hdr, uint64_t* slots, int par,
                                                   int n_tiles, uint64_t max_slots) {
    const int tid = threadIdx.x;
    uint64_t hw = load_agent(&hdr[kHdrHw]);
    if (hw < (uint64_t)n_tiles) hw = (uint64_t)n_tiles;
    if (hw > max_slots) hw = max_slots;
    if (blockIdx.x == 0 && tid == 0) {
        fetch_max_agent(&hdr[kHdrHw], (uint64_t)n_tiles);
        hdr[kHdrT + (par ^ 1)] = 0;
    }
    const int op = par ^ 1;
    for (uint64_t s = (uint64_t)blockIdx.x * kScanThreads + tid; s < hw;
         s += (uint64_t)gridDim.x * kScanThreads) {
        slots[kSlotWords * s + kSlotA + op] = 0;
        slots[kSlotWords * s + kSlotGT + op] = 0;
        slots[kSlotWords * s + kSlotMin + op] = 0;
    }
}

// Wait (wave-wide, bounded) until every lane's needed words are non-zero.
template <int NW>
__device__ __forceinline__ void wait_words(const uint64_t* const (&addr)[NW], const bool (&need)[NW],
                                           uint64_t (&w)[NW], uint64_t* err_word) {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = need[i] ? load_agent(addr[i]) : 0;
    int polls = 0;
    for (;;) {
        bool missing = false;
#pragma unroll
        for (int i = 0; i < NW; ++i) missing = missing || (need[i] && w[i] == 0);
        if (!__any(missing)) break;
        if (++polls > kSpinLimit) {
            if (lane_id() == 0)
                __hip_atomic_fetch_or(err_word, (uint64_t)1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int i = 0; i < NW; ++i)
            if (need[i] && w[i] == 0) w[i] = load_agent(addr[i]);
    }
}

// Serial (left to right) sum of one value per lane, lanes 0..cnt-1, added to f.
template <class Acc>
__device__ __forceinline__ Acc serial_fold(Acc f, Acc x, int cnt) {
    for (int l = 0; l < cnt; ++l) f = f + readlane(x, l);
    return f;
}

// Lookback of one tile, called by wave 0.  Needs the sums A of the earlier
// tiles of its group and the totals GT of the earlier groups; all words are
// requested in one round trip, then folded in a fixed order.  Returns
// excl_j and excl_{j+1} (see the header comment).  The tile that ends a
// group publishes the group total; the last tile advances the call counter.
template <class Acc>
__device__ __forceinline__ void lookback(int tile, int n_tiles, int par, Acc A, uint64_t* slots,
                                         uint64_t* hdr, uint32_t calls, Acc* s_excl) {
    const int lane = threadIdx.x & 63;
    const int g = tile / kScanGroup;
    const int first = g * kScanGroup;
    const int cnt = tile - first;
    Acc F = Acc(0);
    Acc P = Acc(0), Pn = Acc(0);
    bool have_p = false;
    for (int h0 = 0; h0 < g || !have_p; h0 += kGtWords * kWave) {
        const uint64_t* addr[kGtWords + 1];
        bool need[kGtWords + 1];
        uint64_t w[kGtWords + 1];
        addr[0] = slot_word(slots, (uint64_t)(first + lane), kSlotA, par);
        need[0] = !have_p && lane < cnt;
#pragma unroll
        for (int i = 0; i < kGtWords; ++i) {
            const int h = h0 + i * kWave + lane;
            addr[i + 1] = slot_word(slots, (uint64_t)h * kScanGroup, kSlotGT, par);
            need[i + 1] = h < g;
        }
        wait_words<kGtWords + 1>(addr, need, w, &hdr[kHdrErr]);
        if (!have_p) {
            Acc a = Acc(0);
            if (lane < cnt) status_dec(w[0], a);
            P = wave_sum(a);
            Pn = wave_sum(lane == cnt ? A : a);
            have_p = true;
            if (cnt == kScanGroup - 1 && lane == 0)
                store_agent(slot_word(slots, (uint64_t)first, kSlotGT, par), status_enc(P + A));
        }
#pragma unroll
        for (int i = 0; i < kGtWords; ++i) {
            const int base = h0 + i * kWave;
            if (base < g) {
                Acc x = Acc(0);
                if (need[i + 1]) status_dec(w[i + 1], x);
                F = serial_fold(F, x, min_(kWave, g - base));
            }
        }
    }
    if (lane == 0) {
        const Acc excl = F + P;
        // excl of the next tile: same group -> F + P_{j+1}; group end ->
        // F_{g+1} = F_g + GT_g with GT_g = P_j + A_j.
        const Acc next = (cnt < kScanGroup - 1) ? F + Pn : F + (P + A);
        s_excl[0] = excl;
        s_excl[1] = next;
        if (tile == n_tiles - 1) store_agent(&hdr[kHdrCalls], (uint64_t)(calls + 1u));
    }
}

// The tile's CDF values: excl + local prefix; in fp mode made monotone and
// clamped to the next tile's exclusive prefix (see the header comment).
// prepare() runs the block-wide part (one barrier, fp only): pm[r] is the
// max over all tile values before this thread's 4 elements of row r (row-
// major order r, thread, column) -- a thread's own 4 values are ordered, so
// max(value, pm[r]) is the running max.  at() forms one element's value.
template <int R, class Acc>
struct TileValues {
    Acc excl, next;
    bool last;
    double pm[R];

    __device__ __forceinline__ void prepare(const Acc (&q)[R][4], const Acc (&X)[R], Acc excl_,
                                            Acc next_, bool last_, double (*s_wmax)[R]) {
        excl = excl_;
        next = next_;
        last = last_;
        if constexpr (std::is_same<Acc, double>::value) {
            const int tid = threadIdx.x;
            const int wave = tid >> 6;
            const int lane = tid & 63;
            double ex[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                double x = excl + (X[r] + q[r][3]);   // values are >= 0: 0 is the max identity
                x = fmax(x, dpp<kRowShr1, 0xF, true>(x));
                x = fmax(x, dpp<kRowShr2, 0xF, true>(x));
                x = fmax(x, dpp<kRowShr4, 0xF, true>(x));
                x = fmax(x, dpp<kRowShr8, 0xF, true>(x));
                x = fmax(x, dpp<kRowBcast15, 0xA, false>(x));
                x = fmax(x, dpp<kRowBcast31, 0xC, false>(x));
                ex[r] = wave_shr1(x);
                const double wm = readlane(x, kWave - 1);
                if (lane == 0) s_wmax[wave][r] = wm;
            }
            __syncthreads();
            double carry = 0.0;                      // max over earlier rows
#pragma unroll
            for (int r = 0; r < R; ++r) {
                double p = carry, rm = carry;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const double t = s_wmax[w2][r];
                    if (w2 < wave) p = fmax(p, t);
                    rm = fmax(rm, t);
                }
                pm[r] = fmax(p, ex[r]);
                carry = rm;
            }
        }
    }

    __device__ __forceinline__ Acc at(const Acc (&q)[R][4], const Acc (&X)[R], int r, int k) const {
        Acc x = excl + (X[r] + q[r][k]);
        if constexpr (std::is_same<Acc, double>::value) {
            x = fmax(x, pm[r]);
            if (!last) {
                x = fmin(x, next);
                if (r == R - 1 && k == 3 && threadIdx.x == kScanThreads - 1) x = next;
            }
        }
        return x;
    }
};

}  // namespace psamp
