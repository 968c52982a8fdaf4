// scan_tile.h -- the tile machinery shared by the CDF scan and the fused PER
// update: tile loads, weights, the tile-local scan, the fixed-association
// lookback and the monotone tile values.
//
// The CDF of the pages is one serial prefix sum ("trainer: parallel
// build_cdf scan + tiled ... mingru backward", "1. Parallel build_cdf").
// Here it is formed tile by tile (256 threads x 4R elements) in one pass,
// and in fp mode its value does not depend on timing: every partial sum is
// a fixed expression of the tile sums A_j.
//   * Tiles form groups of 64.  P_j (the sum of the earlier tiles of j's
//     group) is the 64-lane DPP tree over A of those tiles (0 in the other
//     lanes); the group total GT_g is the same tree over all 64 tiles.
//   * excl_j = Outer(GT_0, ..., GT_{g-1}, P_j): group h is a leaf in lane
//     h mod 64, slot h / 64; each lane adds its leaves in slot order, then
//     the 64 lane sums go through the DPP tree.  Rounding is monotone and
//     every leaf is >= 0, so excl_j is non-decreasing in j, and
//     excl_{j+1}, computed by tile j (with P_{j+1}, or GT_g at a group end)
//     is bit for bit the value tile j+1 computes.
//   * A tile waits only for sums of tiles near it: it reads A of its own
//     group and of the previous one (and forms GT_{g-1} itself), and the
//     published totals of the groups before that, which are 64 or more tiles
//     older, all in one round trip; no partial sum is folded serially.  (The
//     tile that ends a group publishes GT_g after that round, so each total
//     follows the one two groups before it; publishing it before the round
//     cost that tile a second round trip and measured slower.)
//   * Inside a tile, a running max removes rounding dips between threads;
//     every tile is clamped from above by excl_{j+1} and its last element is
//     set to excl_{j+1}.  So C[end_j - 1] == excl_{j+1} <= C[end_j], the CDF
//     is non-decreasing everywhere, tile j owns exactly the thresholds in
//     (excl_j, excl_{j+1}] (tile 0 from -inf, the last tile up to +inf), and
//     the total T = C_{n-1} is the Outer tree over all group totals, a value
//     any tile that has read every A can form.
// Integer mode is exact and needs none of this, but shares the code.
//
// Workspace: a 256-byte header (call counter, high-water mark, error bits,
// T per parity, a dummy word for polls, the tile-sum pass's exit counter,
// the large fused update's draw-minimum slots per parity), then one 4 KiB
// block per 64 tiles (block b holds the words of tiles 64b..64b+63):
//   [  0,  64) A, parity 0      [ 64, 128) A, parity 1
//   [128, 192) MIN, parity 0    [192, 256) MIN, parity 1
//   [256, 512) group totals GT of groups 128b..128b+127, two parities each
// Consecutive tiles' words are adjacent, so a wave reads 64 of them in a
// few cache lines.  The layout does not depend on n or on the workspace
// size, so a workspace can serve calls of any size.
#pragma once

#include <type_traits>

#include "psamp_device.h"

namespace psamp {

constexpr int kScanThreads = 256;
constexpr int kScanGroup = 64;         // tiles per lookback group (one per lane)
constexpr int kWsHeaderWords = 32;     // 256-byte header
constexpr int kBlockWords = 512;       // status words per 64 tiles
constexpr int kMinTile = kScanThreads * 4;
constexpr int kSpinLimit = 1 << 21;    // bounded waits (about a second)
constexpr int kLbGtWords = 2;          // group totals per lane per round trip (lookback)
constexpr int kAllWords = 4;           // tile sums per lane per round trip (lookback_all)

enum : int {
    kHdrCalls = 0, kHdrHw = 1, kHdrErr = 2, kHdrT = 4, kHdrDummy = 8, kHdrExit = 16,
    kHdrDrawMin = 20     // 2 parities x kDrawMinSlots: max of ~(smallest drawn priority bits)
};
constexpr int kDrawMinSlots = 4;

// Rows of 1024 elements per tile.  The tiling fixes the association of the
// fp sums, so the scan and the fused update both take it from here.
constexpr int64_t kSmallScanN = int64_t(1) << 20;
__host__ __device__ constexpr int scan_rows_for(int64_t n) { return n <= kSmallScanN ? 1 : 8; }

// Bytes of workspace for up to `tiles` tiles, and the tiles a workspace holds.
__host__ __device__ constexpr size_t ws_bytes_for_tiles(int64_t tiles) {
    return (size_t)kWsHeaderWords * 8 +
           (size_t)((tiles + kScanGroup - 1) / kScanGroup) * kBlockWords * 8;
}
__host__ __device__ constexpr uint64_t ws_tile_capacity(size_t ws_bytes) {
    return ws_bytes < (size_t)kWsHeaderWords * 8
               ? 0
               : (uint64_t)((ws_bytes - (size_t)kWsHeaderWords * 8) / (kBlockWords * 8)) *
                     kScanGroup;
}

// Status words are addressed by their word offset from the start of the
// workspace (32 bits: a workspace never holds more than 2^31 / 1024 tiles).
__device__ __forceinline__ uint32_t a_off(uint32_t tile, int par) {
    return kWsHeaderWords + (tile / kScanGroup) * kBlockWords + par * kScanGroup +
           tile % kScanGroup;
}
__device__ __forceinline__ uint32_t min_off(uint32_t tile, int par) {
    return kWsHeaderWords + (tile / kScanGroup) * kBlockWords + 2 * kScanGroup +
           par * kScanGroup + tile % kScanGroup;
}
__device__ __forceinline__ uint32_t gt_off(uint32_t group, int par) {
    return kWsHeaderWords + (group / 128) * kBlockWords + 4 * kScanGroup + 2 * (group % 128) +
           par;
}

template <class In> struct ScanAcc;
template <> struct ScanAcc<float> { using type = double; };
template <> struct ScanAcc<uint32_t> { using type = uint64_t; };

__device__ __forceinline__ double to_weight(float p, double alpha, const MathLds* M) {
    return pow_prio(p, alpha, M);
}
__device__ __forceinline__ uint64_t to_weight(uint32_t q, double, const MathLds*) {
    return (uint64_t)q;
}

// Loads a tile: tin points at the tile's first element, tlen (>= 1) is the
// number of valid elements.  VEC: the input is 16-byte aligned and n % 4 ==
// 0, so every 4-element chunk is wholly valid or wholly invalid and is read
// with one 16-byte load; otherwise element by element.  Invalid elements
// read as 0: every load is issued (from the tile's element 0 when invalid)
// and the value selected afterwards -- a load under a branch would be waited
// for at the end of the branch, one round trip per load.  Offsets are 32-bit
// and tile-local, so the addresses stay a uniform base plus a lane offset.
template <int R, bool VEC, class In>
__device__ __forceinline__ void load_tile(const In* __restrict__ tin, int tlen, In (&v)[R][4]) {
    constexpr int ROW = kScanThreads * 4;
    const int t4 = 4 * (int)threadIdx.x;
    const int lim = tlen - t4;           // element (r, c) is valid iff r*ROW + c < lim
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e0 = r * ROW + t4;
        if constexpr (VEC) {
            const bool ok = r * ROW < lim;
            const uint4 x = *reinterpret_cast<const uint4*>(tin + (ok ? e0 : 0));
            v[r][0] = ok ? __builtin_bit_cast(In, x.x) : In(0);
            v[r][1] = ok ? __builtin_bit_cast(In, x.y) : In(0);
            v[r][2] = ok ? __builtin_bit_cast(In, x.z) : In(0);
            v[r][3] = ok ? __builtin_bit_cast(In, x.w) : In(0);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool ok = r * ROW + c < lim;
                const In e = tin[ok ? e0 + c : 0];
                v[r][c] = ok ? e : In(0);
            }
        }
    }
}

// Zero the other parity's status words (A and MIN of every tile below the
// high-water mark, GT of their groups, and the other T word) so that the
// next call finds them clean.  The high-water mark is the largest tile count
// any call on this workspace has used (hw_seen: its value when the kernel
// started).  Threads t = 0..nt-1 of every workgroup share the work; it is
// done while wave 0 looks back.
__device__ __forceinline__ void clear_other_parity(uint64_t* ws, int par, int n_tiles,
                                                   uint64_t max_tiles, uint64_t hw_seen, int t,
                                                   int nt) {
    uint64_t hw = hw_seen;
    if (hw < (uint64_t)n_tiles) hw = (uint64_t)n_tiles;
    if (hw > max_tiles) hw = max_tiles;
    const int op = par ^ 1;
    if (blockIdx.x == 0 && t == 0) {
        fetch_max_agent(&ws[kHdrHw], (uint64_t)n_tiles);
        ws[kHdrT + op] = 0;
    }
    if (blockIdx.x == 0 && t < kDrawMinSlots) ws[kHdrDrawMin + kDrawMinSlots * op + t] = 0;
    const uint32_t groups = (uint32_t)((hw + kScanGroup - 1) / kScanGroup);
    for (uint32_t s = blockIdx.x * (uint32_t)nt + t; s < hw; s += gridDim.x * (uint32_t)nt) {
        ws[a_off(s, op)] = 0;
        ws[min_off(s, op)] = 0;
        if (s < groups) ws[gt_off(s, op)] = 0;
    }
}

// Wait (wave-wide, bounded) until every lane's needed words ws[off[i]] are
// non-zero.  Words that are not needed are set to 1, which decodes to 0 in
// both status encodings.  Two polls are kept in flight: the next one is
// issued before the previous one is examined, which halves the time between
// a word being published and the wave seeing it.  A lane whose word is
// already known (or not needed) reads a dummy header word that all such
// lanes share, so the loop has no per-word branch.
template <int NW>
__device__ __forceinline__ void wait_words(const uint64_t* ws, const uint32_t (&off)[NW],
                                           const bool (&need)[NW], uint64_t (&w)[NW]) {
    uint64_t a[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        a[i] = load_agent(&ws[need[i] ? off[i] : (uint32_t)kHdrDummy]);
        w[i] = need[i] ? 0 : 1;
    }
    // The bound is hidden from the optimiser: with a known trip count it
    // unrolls the poll loop into a hundred copies.
    int limit = kSpinLimit;
    asm volatile("" : "+s"(limit));
    int polls = 0;
    for (;;) {
        uint64_t b[NW];
        for (int i = 0; i < NW; ++i)
            b[i] = load_agent(&ws[w[i] == 0 ? off[i] : (uint32_t)kHdrDummy]);
        bool missing = false;
        for (int i = 0; i < NW; ++i) {
            w[i] = w[i] == 0 ? a[i] : w[i];
            missing = missing || w[i] == 0;
        }
        if (!__any(missing)) break;
        if (++polls > limit) {
            if (lane_id() == 0)
                __hip_atomic_fetch_or(const_cast<uint64_t*>(&ws[kHdrErr]), (uint64_t)1,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        for (int i = 0; i < NW; ++i) a[i] = b[i];
    }
}

template <class Acc>
__device__ __forceinline__ Acc status_value(uint64_t w) {
    Acc x;
    status_dec(w, x);
    return x;
}

// The words of the first lookback round of a tile (see lookback): A of
// every tile of the previous group (slot 0), A of the earlier tiles of its
// own group (slot 1), the published totals GT_h of groups h < g - 1, 64 per
// slot (slots 2..).  Words not needed are marked so.
__device__ __forceinline__ void lb_round(int tile, int par, int s0, uint32_t (&off)[kLbGtWords + 2],
                                         bool (&need)[kLbGtWords + 2]) {
    const int lane = threadIdx.x & 63;
    const int g = tile / kScanGroup;
    const int cnt = tile - g * kScanGroup;
    const int gp = g > 0 ? g - 1 : 0;
    const bool first = s0 == 0;
    need[0] = first && g > 0;
    off[0] = a_off((uint32_t)(gp * kScanGroup + lane), par);
    need[1] = first && lane < cnt;
    off[1] = a_off((uint32_t)(g * kScanGroup + lane), par);
#pragma unroll
    for (int i = 0; i < kLbGtWords; ++i) {
        const int h = (s0 + i) * kWave + lane;
        need[i + 2] = h < g - 1;
        off[i + 2] = gt_off((uint32_t)(need[i + 2] ? h : 0), par);
    }
}

// Issues the loads of the first lookback round ahead of time (wave 0, when
// every sum is known to be published already: the second pass of a
// reduce-then-scan); lookback<Acc, true> then uses them instead of polling.
__device__ __forceinline__ void lb_preload(int tile, int par, const uint64_t* ws,
                                           uint64_t (&pre)[kLbGtWords + 2]) {
    uint32_t off[kLbGtWords + 2];
    bool need[kLbGtWords + 2];
    lb_round(tile, par, 0, off, need);
#pragma unroll
    for (int i = 0; i < kLbGtWords + 2; ++i) pre[i] = load_agent(&ws[need[i] ? off[i] : kHdrDummy]);
}

// Lookback of one tile, called by wave 0 after the tile published its sum
// A.  Reads A of the earlier tiles of its group and of the whole previous
// group, and the published totals GT_h of the groups h < g - 1, all in one
// round trip (more only past 64 * kLbGtWords groups); forms P_j, P_{j+1},
// GT_{g-1} and the two Outer trees of the header comment.  Writes excl_j to
// s_excl[0] and excl_{j+1} to s_excl[1].  The tile that ends a group
// publishes GT_g; the last tile advances the call counter -- by then every
// workgroup has read it, since the last tile's lookback needs every tile's
// sum.  PRE: the first round's words were loaded by lb_preload; they are
// used if every needed one is there (otherwise the round polls as usual).
// A PRE lookback does not advance the counter: its tiles' sums were
// published by an earlier kernel, so the last tile can finish before other
// workgroups have even started (the earlier kernel advances it instead).
template <class Acc, bool PRE = false>
__device__ __forceinline__ void lookback(int tile, int n_tiles, int par, Acc A, uint64_t* ws,
                                         uint32_t calls, Acc* s_excl,
                                         const uint64_t* pre = nullptr) {
    const int lane = threadIdx.x & 63;
    const int g = tile / kScanGroup;
    const int cnt = tile - g * kScanGroup;
    Acc base = Acc(0);     // this lane's published leaves h < g - 1, in slot order
    Acc P = Acc(0), Pn = Acc(0), Gp = Acc(0);
#pragma nounroll
    for (int s0 = 0;; s0 += kLbGtWords) {
        const bool first = s0 == 0;
        uint32_t off[kLbGtWords + 2];
        bool need[kLbGtWords + 2];
        uint64_t w[kLbGtWords + 2];
        lb_round(tile, par, s0, off, need);
        bool have = false;
        if constexpr (PRE) {
            if (first) {
                bool miss = false;
#pragma unroll
                for (int i = 0; i < kLbGtWords + 2; ++i) {
                    w[i] = pre[i];
                    miss = miss || (need[i] && w[i] == 0);
                }
                have = !__any(miss);
            }
        }
        if (!have) wait_words<kLbGtWords + 2>(ws, off, need, w);
        if (first) {
            // P_j, P_{j+1} and GT_{g-1}, formed together
            const Acc a = need[1] ? status_value<Acc>(w[1]) : Acc(0);
            Acc x[3] = {a, lane == cnt ? A : a,
                        (g > 0 && need[0]) ? status_value<Acc>(w[0]) : Acc(0)};
            wave_sums(x);
            P = x[0];
            Pn = x[1];
            if (cnt == kScanGroup - 1 && lane == 0)
                store_agent(&ws[gt_off((uint32_t)g, par)], status_enc(Pn));
            if (g > 0) Gp = x[2];
        }
#pragma unroll
        for (int i = 0; i < kLbGtWords; ++i)
            if (need[i + 2]) base = base + status_value<Acc>(w[i + 2]);
        if ((s0 + kLbGtWords) * kWave >= g - 1) break;
    }
    if (g > 0 && lane == (g - 1) % kWave) base = base + Gp;
    const bool mine = lane == g % kWave;
    Acc y[2] = {mine ? base + P : base, mine ? base + Pn : base};
    wave_sums(y);                       // excl_j, excl_{j+1}
    if (lane == 0) {
        s_excl[0] = y[0];
        s_excl[1] = y[1];
        if (!PRE && tile == n_tiles - 1) store_agent(&ws[kHdrCalls], (uint64_t)(calls + 1u));
    }
}

// Lookback of a tile when the whole grid is resident (the fused update):
// every tile reads the sums A of all tiles (kAllWords groups per round trip),
// forms every group total GT_h itself and writes excl_j, excl_{j+1} and the
// total T = Outer(GT_0, ..., GT_{G-1}) to s_out[0..2].  The association is
// that of lookback() (lane h mod 64 adds its leaves in increasing h, then
// the DPP tree), so excl_j and excl_{j+1} are bit for bit the values the
// standalone scan forms, and T equals the scan's C_{n-1}.  No hop through
// the last tile is needed to learn T.
template <class Acc>
__device__ __forceinline__ void lookback_all(int tile, int n_tiles, int par, Acc A, uint64_t* ws,
                                             uint32_t calls, Acc* s_out) {
    const int lane = threadIdx.x & 63;
    const int g = tile / kScanGroup;
    const int cnt = tile - g * kScanGroup;
    const int G = (n_tiles + kScanGroup - 1) / kScanGroup;
    Acc accx = Acc(0);     // this lane's leaves h < g, in increasing h
    Acc acct = Acc(0);     // this lane's leaves h < G
    Acc P = Acc(0), Pn = Acc(0);
#pragma nounroll
    for (int h0 = 0; h0 < G; h0 += kAllWords) {
        uint32_t off[kAllWords];
        bool need[kAllWords];
        uint64_t w[kAllWords];
#pragma unroll
        for (int i = 0; i < kAllWords; ++i) {
            const int t = (h0 + i) * kScanGroup + lane;
            need[i] = t < n_tiles && t != tile;
            off[i] = a_off((uint32_t)(need[i] ? t : 0), par);
        }
        wait_words<kAllWords>(ws, off, need, w);
        // the round's group totals (and P_j, P_{j+1} when g is among them),
        // formed together
        Acc x[kAllWords + 2];
        const int ig = g - h0;             // g's slot in this round, if any
#pragma unroll
        for (int i = 0; i < kAllWords; ++i) {
            Acc a = need[i] ? status_value<Acc>(w[i]) : Acc(0);
            if (i == ig) {
                if (lane == cnt) a = A;
                const Acc below = lane < cnt ? a : Acc(0);
                x[kAllWords] = below;
                x[kAllWords + 1] = lane == cnt ? a : below;
            }
            x[i] = a;
        }
        if (ig < 0 || ig >= kAllWords) x[kAllWords] = x[kAllWords + 1] = Acc(0);
        wave_sums(x);
        if (ig >= 0 && ig < kAllWords) {
            P = x[kAllWords];
            Pn = x[kAllWords + 1];
        }
#pragma unroll
        for (int i = 0; i < kAllWords; ++i) {
            const int h = h0 + i;
            if (h < G && lane == h % kWave) {
                if (h < g) accx = accx + x[i];
                acct = acct + x[i];
            }
        }
    }
    const bool mine = lane == g % kWave;
    Acc y[3] = {mine ? accx + P : accx, mine ? accx + Pn : accx, acct};
    wave_sums(y);                       // excl_j, excl_{j+1}, T
    if (lane == 0) {
        s_out[0] = y[0];
        s_out[1] = y[1];
        s_out[2] = y[2];
        if (tile == n_tiles - 1) store_agent(&ws[kHdrCalls], (uint64_t)(calls + 1u));
    }
}

// The tile's local values, in place.  On entry q[r][c] is the prefix of the
// thread's 4 elements of row r and X[r] the sum of the tile's elements
// before them; on exit q[r][c] = fl(X[r] + q[r][c]), and in fp mode also
// raised to the running max of all local values before it in memory order
// (rows, then threads, then columns; a thread's own 4 values are already
// ordered).  fl(excl + x) is non-decreasing in x, so raising the local
// values before adding excl gives the same bits as raising the sums:
// max_i fl(excl + x_i) = fl(excl + max_i x_i).  One barrier (fp only); runs
// before the lookback, so only q stays live across it.
template <int R, class Acc>
__device__ __forceinline__ void tile_local_values(Acc (&q)[R][4], const Acc (&X)[R],
                                                  double (*s_wmax)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) q[r][c] = X[r] + q[r][c];
    if constexpr (std::is_same<Acc, double>::value) {
        const int tid = threadIdx.x;
        const int wave = tid >> 6;
        const int lane = tid & 63;
        double ex[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            double x = q[r][3];                       // values are >= 0: 0 is the max identity
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
        double carry = 0.0;                          // max over earlier rows
#pragma unroll
        for (int r = 0; r < R; ++r) {
            double p = carry, rm = carry;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const double t = s_wmax[w2][r];
                if (w2 < wave) p = fmax(p, t);
                rm = fmax(rm, t);
            }
            const double pm = fmax(p, ex[r]);
#pragma unroll
            for (int c = 0; c < 4; ++c) q[r][c] = fmax(q[r][c], pm);
            carry = rm;
        }
    }
}

// One CDF value from a local value x (see tile_local_values): excl + x, in
// fp mode clamped to excl_{j+1}; the tile's last valid element is
// excl_{j+1} itself, so in the last tile C_{n-1} = T is the Outer tree over
// all group totals.
template <class Acc>
__device__ __forceinline__ Acc tile_value(Acc x, Acc excl, Acc next, bool last_e) {
    if constexpr (std::is_same<Acc, double>::value) {
        const double y = fmin(excl + x, next);
        return last_e ? next : y;
    } else {
        return excl + x;
    }
}

// ------------------------------------------- stratified draws of a tile
// Stratified threshold of draw i (the same operations as psamp_sample):
// fl(fl(fl(i + u) / k) * T).  For a power-of-two k the division is the
// multiplication by inv_k = 1/k (exact, so the same bits), which spares the
// long chain of a double divide on the path to the draws.
struct KDiv {
    int64_t k;
    double inv_k;
    bool pow2;
    __device__ __forceinline__ explicit KDiv(int64_t k_)
        : k(k_), inv_k(1.0 / (double)k_), pow2((k_ & (k_ - 1)) == 0) {}
    __device__ __forceinline__ double div(double a) const {
        return pow2 ? a * inv_k : a / (double)k;
    }
};
__device__ __forceinline__ double strat_threshold(int64_t i, float u, const KDiv& kd, double T) {
    const double a = (double)i + (double)u;
    const double b = kd.div(a);
    return b * T;
}

// t_i for fp and integer mode (integer: the exact map onto [1, T]).
struct StratFp {
    const float* U;
    KDiv kd;
    double T;
    __device__ __forceinline__ double operator()(int64_t i) const {
        return strat_threshold(i, U[i], kd, T);
    }
};
struct StratInt {
    const uint32_t* r;
    int64_t k;
    uint64_t T;
    int k_log2;
    __device__ __forceinline__ uint64_t operator()(int64_t i) const {
        return int_threshold((uint64_t)i, r[i], (uint64_t)k, T, 1, k_log2);
    }
};

// First i in [0, k] with t_i > B (t_i non-decreasing in i).  Lanes 0..31
// answer for B0, lanes 32..63 for B1, in one round trip: each half tests a
// 32-wide window around the stratum estimate B k / T (the answer lies within
// 2 of it); a binary search covers the case the window misses (T = 0, or
// inputs outside the preconditions).  With the exactly monotone CDF, tile j
// owns the draws [first_above(excl_j), first_above(excl_{j+1})).
template <class Thr, class V>
__device__ __forceinline__ int64_t first_above2(V B0, V B1, V T, const Thr& thr, int64_t k) {
    const int lane = lane_id();
    const bool hi = lane >= 32;
    const V B = hi ? B1 : B0;
    int64_t est = 0;
    if (T > V(0)) {
        const double e = floor((double)B / (double)T * (double)k);
        est = !(e > 0.0) ? 0 : (e > (double)k ? k : (int64_t)e);
    }
    const int64_t c0 = est - 8;
    const int64_t c = c0 + (lane & 31);
    const bool above = c < 0 ? false : (c >= k ? true : thr(c) > B);
    const uint64_t bal = __ballot(above);
    const uint32_t m = hi ? (uint32_t)(bal >> 32) : (uint32_t)bal;
    if (m != 0 && ((m & 1u) == 0 || c0 <= 0)) {
        const int64_t r = c0 + (__ffs((int)m) - 1);
        return r < 0 ? 0 : r;
    }
    int64_t lo = 0, hi_i = k;
    while (lo < hi_i) {
        const int64_t mid = lo + ((hi_i - lo) >> 1);
        if (thr(mid) > B) hi_i = mid;
        else lo = mid + 1;
    }
    return lo;
}

}  // namespace psamp
