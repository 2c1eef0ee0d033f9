// sad_propagate.h -- one top-K propagation pass (Sec. 4.3, Figure 5) over
// one pixel tile, as a device function shared by the propagation kernel and
// the fused last-pass + backward kernel.
//
// Mapping: one wavefront (64 lanes) per 8x8 pixel tile, one lane per pixel.
// The tile is also the unit of the global probe: its injected ids are drawn
// once per wavefront, one per lane, and shared by all pixels of the tile.
//
// Work per lane, in the order that keeps the vector ALU busy the least:
//  1. The pixel's previous list: 8 logits (or the caller's score map), then
//     a sorting network puts the entries in ranking order (a list carried
//     over from the previous pass is already in order unless the sites moved,
//     and the network is skipped when every lane of the wavefront is in
//     order).
//  2. The neighbour lists, two at a time (16 ids): each id is compared with
//     the ids now in the pixel's list and only ids not already listed are
//     queued, in LDS (one column per lane).  At small strides almost all
//     neighbour ids are already listed.  The queued ids are scored against
//     the list's current 8th entry; the few that beat it are compacted, with
//     their logits, to the front of the column and then inserted.  Keeping
//     insertion out of the scoring loop leaves that loop free of divergent
//     updates of the list.
//  3. The tile's probe ids: each lane bounds its probe site's logit over the
//     whole tile (probe_may_enter) and the wavefront scores only the sites
//     whose bound can beat the tile's weakest 8th entry.
// The result equals the top-8 of the candidate set in ranking order, whatever
// order the candidates are visited in: every step above only skips
// candidates that provably cannot be among the 8 best (the 8th entry only
// improves as candidates are inserted).
#pragma once

#include <type_traits>

#include "sad_device.h"
#include "sad_host.h"

namespace sad {

struct PropArgs {
    const float* derived;
    const uint32_t* prev;      // the previous map with 32-bit ids, or
    const uint16_t* prev16;    // with 16-bit ids (at most one of the two; neither: an empty map)
    const float* prev_scores;  // nullable: logits of prev's entries under derived
    const float* prev_thr;     // nullable (not with prev_scores): the logit of each prev list's 8th entry
    uint32_t* next;            // the next map with 32-bit ids, or
    uint16_t* next16;          // with 16-bit ids (exactly one of the two)
    float* next_scores;        // nullable: logits of next's entries are written here
    float* next_thr;           // nullable: the logit of each next list's 8th entry is written here
    const float4* probe_prev;  // nullable: the sites' probe records (probe_record), for the tile cull
    float4* probe_next;        // nullable: the sites' probe records are written here
    uint64_t seed;
    int32_t n, h, w, stride, inject, tiles_x, n_tiles;
    uint32_t pass_index;
};

constexpr int QCAP = 2 * K;  // queued neighbour ids per lane (2 lists of 8)

// Can the probe site (geometry g) rank among the 8 best of any pixel of the
// tile whose pixel centres span [bx0, bx1] x [by0, by1], given that every
// pixel of the tile already holds 8 entries of logit >= thr?
//
// For every pixel centre P of the box, ||P - p||_G >= m ||P - p||_2 >= m D,
// with m the smaller inverse scale and D the distance from p to the box, so
// the exact logit is at most -tau (m D - r).  The float32 evaluation of the
// logit differs from the exact one by at most tau u ((8.5 kappa + 4) sqrt(q)
// + 2 |r|), u = 2^-24, kappa = M/m the anisotropy ratio; for kappa <= 1024
// this is below 2^-8 (tau sqrt(q) + tau |r|).  The bound therefore keeps a
// 2^-8 relative margin on both terms, which also covers the rounding of the
// bound's own evaluation.  Sites with non-finite values, tau <= 0 (a logit
// that does not fall with distance) or extreme anisotropy are never culled.
__device__ __forceinline__ bool probe_may_enter(const Geo& g, float thr, float bx0, float bx1, float by0,
                                                float by1) {
    float tau = g.g0.z, r = g.g0.w, is1 = g.g1.z, is2 = g.g1.w;
    float m = fminf(is1, is2), M = fmaxf(is1, is2);
    const bool fin_x = finitef(g.g0.x), fin_y = finitef(g.g0.y), fin_tau = finitef(tau), fin_r = finitef(r),
               fin_m = finitef(M);
    const bool boundable = fin_x & fin_y & fin_tau & fin_r & fin_m & (tau > 0.0f) & (m > 0.0f) & (M <= 1024.0f * m);
    float ex = fmaxf(fmaxf(bx0 - g.g0.x, g.g0.x - bx1), 0.0f);
    float ey = fmaxf(fmaxf(by0 - g.g0.y, g.g0.y - by1), 0.0f);
    float dist = __builtin_sqrtf(ex * ex + ey * ey);
    float A = tau * (m * dist);
    float C = tau * r;
    float ub = (C - A * (1.0f - 0x1p-8f)) + 0x1p-8f * (tau * fabsf(r));
    return !boundable | !(ub < thr);  // values of an unboundable site are not used
}

// probe_may_enter from a probe record: the same bound with tau m and tau r
// rounded once more (a few float32 roundings, far inside its 2^-8 margin);
// an unboundable site's infinite tau r passes, as does anything NaN.
__device__ __forceinline__ bool probe_record_may_enter(const float4 pr, float thr, float bx0, float bx1, float by0,
                                                       float by1) {
    const float ex = fmaxf(fmaxf(bx0 - pr.x, pr.x - bx1), 0.0f);
    const float ey = fmaxf(fmaxf(by0 - pr.y, pr.y - by1), 0.0f);
    const float dist = __builtin_sqrtf(ex * ex + ey * ey);
    const float A = pr.z * dist, C = pr.w;
    const float ub = (C - A * (1.0f - 0x1p-8f)) + 0x1p-8f * fabsf(C);
    return !(ub < thr);
}

// A cheap screen in front of the exact logit of a queued neighbour id: false
// only when the float32 logit `logit(g, px, py)` of the site is certainly
// below ts, the logit of the list's 8th entry, so that the site cannot rank
// before that entry; true for an inactive-site test that passes and for
// anything non-finite.  On a settled map almost every queued id is such a
// clear loser, and the screen costs about half of the exact evaluation (no
// correctly rounded square root, fused multiply-adds).
//
// It evaluates l' = tau (r - s') with a' = fma(dx, cos, dy sin) / s1,
// b' = fma(dy, cos, -(dx sin)) / s2, q' = fma(a', a', b'^2) and s' the
// hardware square root of q' (within 1 ulp of the correctly rounded one for
// normal q'), and passes unless l' + M < ts for
//     M = tau (2^-20 (T + 2 (s' + |r|)) + 2^-60),  T = (|dx| + |dy|)(1/s1 + 1/s2).
// Why M bounds |l - l'|, with u = 2^-24, D = |dx| + |dy| and (A, B) the
// rotated, scaled offset in real arithmetic on the same float32 inputs
// (|cos|, |sin| <= 1): both evaluations form a and b within (2u + u^2) D / s_i
// + u |a| (resp. |b|) of A and B, so the two vectors (a, b) lie within
// 2.01 u T + 1.42 u |(a, b)| of (A, B); the squares and their sum scale the
// squared norm by at most 1 + 2u + u^2, i.e. the root by 1 + 1.01 u; the
// correctly rounded root adds u sqrt(q), the hardware one 2u sqrt(q'), so the
// two roots differ by at most 4.02 u T + 8.5 u S (S the larger root).  The
// subtraction of r adds u |d| + u |d'| <= 2u (S + |r|)(1 + u), and the product
// with tau one rounding u |l| <= u tau (S + |r|)(1 + u) on each side, so
// |l - l'| <= tau u (4.02 T + 12.6 S + 4.1 |r|), which M (16 u T + 32 u s'
// + 32 u |r|) exceeds with room for the roundings of M and of l' + M (a
// rounded sum below the float ts implies the exact sum below it).  The last
// term of M covers roots of subnormal q, where the hardware root is only
// absolutely close (sqrt of 2^-126 is 2^-63).
__device__ __forceinline__ bool may_rank_before(const Geo& g, float px, float py, float ts) {
    const float dx = px - g.g0.x, dy = py - g.g0.y;
    const float a = __builtin_fmaf(dx, g.g1.x, dy * g.g1.y) * g.g1.z;
    const float b = __builtin_fmaf(dy, g.g1.x, -(dx * g.g1.y)) * g.g1.w;
    const float q = __builtin_fmaf(a, a, b * b);
    const float s = __builtin_amdgcn_sqrtf(q);
    const float tau = g.g0.z, r = g.g0.w;
    const float l = tau * (r - s);
    const float T = (fabsf(dx) + fabsf(dy)) * (g.g1.z + g.g1.w);
    const float M = tau * __builtin_fmaf(0x1p-20f, __builtin_fmaf(2.0f, s + fabsf(r), T), 0x1p-60f);
    return (g.g0.x >= 0.0f) & !(l + M < ts);
}

// compare-exchange for the sorting network: entry i ends up ranking before j
__device__ __forceinline__ void cex(TopK& t, int i, int j) {
    bool sw = ranks_before(t.s[j], t.id[j], t.s[i], t.id[i]);
    float si = t.s[i], sj = t.s[j];
    uint32_t ii = t.id[i], ij = t.id[j];
    t.s[i] = sw ? sj : si;
    t.s[j] = sw ? si : sj;
    t.id[i] = sw ? ij : ii;
    t.id[j] = sw ? ii : ij;
}

__device__ __forceinline__ void sort8(TopK& t) {
    cex(t, 0, 2); cex(t, 1, 3); cex(t, 4, 6); cex(t, 5, 7);
    cex(t, 0, 4); cex(t, 1, 5); cex(t, 2, 6); cex(t, 3, 7);
    cex(t, 0, 1); cex(t, 2, 3); cex(t, 4, 5); cex(t, 6, 7);
    cex(t, 2, 4); cex(t, 3, 5);
    cex(t, 1, 4); cex(t, 3, 6);
    cex(t, 1, 2); cex(t, 3, 4); cex(t, 5, 6);
}

constexpr int QBATCH = 3;  // queued ids scored per loop trip (their gathers overlap)

// Largest site count for which every usable id fits in 16 bits and differs
// from the low half of EMPTY.
constexpr int32_t SMALL_IDS_MAX = 0xFFFF;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Two ids in the halves of one register (a in the low half), each clamped to
// 0xFFFF: an id >= 2^16 becomes 0xFFFF, which is >= n and is never a usable
// id when n <= SMALL_IDS_MAX.
__device__ __forceinline__ uint32_t pack16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_u16(a, b));
}

// Which of 16 packed ids (pairs[j] holds ids 2j and 2j + 1, as pack16 makes
// them) are in the list t?  Each pair is compared with every list id copied
// into both halves; a packed 16-bit minimum of the differences answers for
// both ids at once.  Only meaningful for ids < n <= SMALL_IDS_MAX (the list
// holds such ids or EMPTY).
__device__ __forceinline__ void listed16(const TopK& t, const uint32_t (&pairs)[K], bool (&in)[2 * K]) {
    uint32_t rep[K];
#pragma unroll
    for (int k = 0; k < K; ++k) rep[k] = __builtin_amdgcn_perm(t.id[k], t.id[k], 0x01000100u);
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const uint32_t pr = pairs[j];
        u16x2 m = __builtin_bit_cast(u16x2, pr ^ rep[0]);
#pragma unroll
        for (int k = 1; k < K; ++k) m = __builtin_elementwise_min(m, __builtin_bit_cast(u16x2, pr ^ rep[k]));
        in[2 * j] = m.x == 0;
        in[2 * j + 1] = m.y == 0;
    }
}

// Queue entry type: 16-bit ids when they fit.
template <bool SMALL_IDS>
using QueueId = std::conditional_t<SMALL_IDS, uint16_t, uint32_t>;

// One propagation pass over one 8x8 tile (tile < a.n_tiles), one lane of the
// calling wavefront per pixel.  queue and qscore are this wavefront's LDS
// columns (QCAP rows of WAVE).  Writes the pixel's new list (and its logits
// when a.next_scores is set) and leaves it in t, in ranking order.  No
// workgroup barrier inside.  SMALL_IDS requires a.n <= SMALL_IDS_MAX; the
// neighbour lists are then held as packed 16-bit pairs and queued as 16-bit
// ids, which leaves registers and LDS for more wavefronts per compute unit.
// PREV16 / NEXT16 (SMALL_IDS only): the previous / next map holds 16-bit ids
// (a.prev16 / a.next16, 16 bytes per pixel, the empty slot 0xffff).  A
// 16-bit list is read as the packed pairs the neighbour lists use anyway,
// and its 0xffff slots, being >= n, are dropped like any unusable id.
// THR_IN: the previous lists come with only their 8th entry's logit
// (a.prev_thr), written by a pass over the same sites, so that they hold
// usable ids in ranking order.  A lane then knows the one logit the screen
// and the ranking against the 8th entry use; the other seven are evaluated
// (materialize) only when the lane is about to insert a candidate or the
// caller asks for all logits, so that a pass on settled lists (almost no
// insertions) reads 4 instead of 32 bytes of logits per pixel.  *lazy (when
// given) receives whether the lane's logits other than the 8th are still
// unknown when the pass ends.
template <bool SMALL_IDS, bool PREV16 = false, bool NEXT16 = false, bool THR_IN = false>
__device__ __forceinline__ void propagate_tile(const PropArgs& a, int tile, QueueId<SMALL_IDS> (*queue)[WAVE],
                                               float (*qscore)[WAVE], TopK& t, bool* lazy_out = nullptr) {
    static_assert(SMALL_IDS || !(PREV16 || NEXT16), "16-bit maps hold 16-bit ids");
    const bool has_prev = PREV16 ? a.prev16 != nullptr : a.prev != nullptr;  // uniform
    constexpr int NW = SMALL_IDS ? K / 2 : K;  // registers per neighbour list
    const int lane = threadIdx.x & (WAVE - 1);
    const int tx = tile % a.tiles_x, ty = tile / a.tiles_x;
    const int i = tx * TILE + (lane & (TILE - 1));
    const int j = ty * TILE + (lane / TILE);
    const bool inside = (i < a.w) & (j < a.h);
    const float px = (float)i + 0.5f, py = (float)j + 0.5f;
    const uint32_t n = (uint32_t)a.n;
    const bool have_prev = inside && has_prev;

    // the sites' probe records for later passes: the wavefront of tile T writes
    // those of sites 64 T + lane, 64 (T + n_tiles) + lane, ...
    if (a.probe_next) {
        for (int64_t si = (int64_t)tile * WAVE + lane; si < a.n; si += (int64_t)a.n_tiles * WAVE)
            a.probe_next[si] = probe_record(load_geo(a.derived, (uint32_t)si));
    }

    // Issue every independent load first: the pixel's list, the 4 neighbour
    // lists and this lane's probe site.  Every list load reads a pixel inside
    // the image (coordinates clamped), so no load waits on a branch; nb_ok
    // marks the neighbours that exist, and a lane off the image uses no list.
    uint32_t own[K];
    float own_s[K];
    uint32_t nbr[4][NW];  // ids, or pack16 pairs of ids
    bool nb_ok[4];
    const int nb[4][2] = {{a.stride, 0}, {-a.stride, 0}, {0, a.stride}, {0, -a.stride}};
    if (has_prev) {  // uniform
        const size_t pc = (size_t)min(j, a.h - 1) * a.w + min(i, a.w - 1);
        if constexpr (PREV16) {
            const uint4 l = *reinterpret_cast<const uint4*>(a.prev16 + pc * K);
            const uint32_t pr[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
            for (int k = 0; k < K / 2; ++k) {
                own[2 * k] = pr[k] & 0xFFFFu;
                own[2 * k + 1] = pr[k] >> 16;
            }
        } else {
            const uint4* l = reinterpret_cast<const uint4*>(a.prev + pc * K);
            const uint4 l0 = l[0], l1 = l[1];
            own[0] = l0.x; own[1] = l0.y; own[2] = l0.z; own[3] = l0.w;
            own[4] = l1.x; own[5] = l1.y; own[6] = l1.z; own[7] = l1.w;
        }
        if constexpr (THR_IN) {
            own_s[K - 1] = a.prev_thr[pc];
        } else if (a.prev_scores) {
            const float4* ls = reinterpret_cast<const float4*>(a.prev_scores + pc * K);
            const float4 s0 = ls[0], s1 = ls[1];
            own_s[0] = s0.x; own_s[1] = s0.y; own_s[2] = s0.z; own_s[3] = s0.w;
            own_s[4] = s1.x; own_s[5] = s1.y; own_s[6] = s1.z; own_s[7] = s1.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ii = i + nb[q][0], jj = j + nb[q][1];
            nb_ok[q] = inside & (ii >= 0) & (ii < a.w) & (jj >= 0) & (jj < a.h);
            const size_t pq = (size_t)min(max(jj, 0), a.h - 1) * a.w + min(max(ii, 0), a.w - 1);
            if constexpr (PREV16) {
                const uint4 m = *reinterpret_cast<const uint4*>(a.prev16 + pq * K);
                nbr[q][0] = m.x; nbr[q][1] = m.y; nbr[q][2] = m.z; nbr[q][3] = m.w;
                continue;
            }
            const uint4* m = reinterpret_cast<const uint4*>(a.prev + pq * K);
            const uint4 m0 = m[0], m1 = m[1];
            if constexpr (SMALL_IDS) {
                nbr[q][0] = pack16(m0.x, m0.y); nbr[q][1] = pack16(m0.z, m0.w);
                nbr[q][2] = pack16(m1.x, m1.y); nbr[q][3] = pack16(m1.z, m1.w);
            } else {
                nbr[q][0] = m0.x; nbr[q][1] = m0.y; nbr[q][2] = m0.z; nbr[q][3] = m0.w;
                nbr[q][4] = m1.x; nbr[q][5] = m1.y; nbr[q][6] = m1.z; nbr[q][7] = m1.w;
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) own[k] = inside ? own[k] : EMPTY;
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) own[k] = EMPTY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            nb_ok[q] = false;
#pragma unroll
            for (int k = 0; k < NW; ++k) nbr[q][k] = EMPTY;
        }
    }
    uint32_t pid = EMPTY;
    if (lane < a.inject) pid = probe_id(a.seed, a.pass_index, (uint32_t)tile, (uint32_t)lane, n);

    // 1. the pixel's previous list, in ranking order (its logits come from the
    //    caller's score map when the sites have not changed since it was made)
    t.clear();
    bool lazy = false;  // THR_IN: the lane's logits other than the 8th are not evaluated yet
    if constexpr (THR_IN) {
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (have_prev & (own[k] < n)) t.id[k] = own[k];
        if (have_prev & (own[K - 1] < n)) t.s[K - 1] = own_s[K - 1];
        lazy = have_prev & (own[0] < n);
    } else if (a.prev_scores) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (have_prev & (own[k] < n) & (own_s[k] == own_s[k])) {
                t.s[k] = own_s[k];
                t.id[k] = own[k];
            }
        }
    } else if (n > 0) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            Geo og[K / 2];
#pragma unroll
            for (int k = 0; k < K / 2; ++k) og[k] = load_geo_clamped(a.derived, n, own[half * 4 + k]);
#pragma unroll
            for (int k = 0; k < K / 2; ++k) {
                const int kk = half * 4 + k;
                const float s = usable_logit(og[k], own[kk] < n, px, py);
                if (s == s) {
                    t.s[kk] = s;
                    t.id[kk] = own[kk];
                }
            }
        }
    }
    // the logits of the lanes in `need` that are still unknown (THR_IN), in
    // the list's order: the same float32 values the pass that wrote the list
    // evaluated
    auto materialize = [&](bool need) {
        if constexpr (THR_IN) {
            need &= lazy;
            if (__any(need)) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    Geo og[K / 2];
#pragma unroll
                    for (int k = 0; k < K / 2; ++k)
                        og[k] = load_geo_clamped(a.derived, n, need ? t.id[half * 4 + k] : EMPTY);
#pragma unroll
                    for (int k = 0; k < K / 2; ++k) {
                        const int kk = half * 4 + k;
                        const float s = usable_logit(og[k], t.id[kk] < n, px, py);
                        t.s[kk] = (need & (t.id[kk] < n)) ? s : t.s[kk];
                    }
                }
                lazy &= !need;
            }
        }
    };
    bool ordered = true;
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
        ordered &= ranks_before(t.s[k], t.id[k], t.s[k + 1], t.id[k + 1]) | (t.id[k + 1] == EMPTY);
    if (THR_IN) ordered = true;  // lists a pass wrote over the same sites are in order
    if (!__all(ordered)) {
        sort8(t);
        // a malformed previous list may repeat an id: rebuild such lists by insertion
        bool dup = false;
#pragma unroll
        for (int k = 0; k < K - 1; ++k) dup |= (t.id[k] == t.id[k + 1] && t.id[k] != EMPTY);
        if (__any(dup)) {
            TopK u;
            u.clear();
#pragma unroll
            for (int k = 0; k < K; ++k) u.insert_if(t.s[k], t.id[k], t.id[k] != EMPTY);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                t.s[k] = dup ? u.s[k] : t.s[k];
                t.id[k] = dup ? u.id[k] : t.id[k];
            }
        }
    }

    // 2. the neighbour lists, two at a time
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        // ids not in the pixel's list go to this lane's queue column; every id
        // is written at the current end of the column and kept only if fresh
        // (the write index never passes the id's own position)
        bool listed[2 * K];
        if constexpr (SMALL_IDS) {
            uint32_t pairs[K];
#pragma unroll
            for (int k = 0; k < K; ++k) pairs[k] = nbr[2 * half + k / NW][k % NW];
            listed16(t, pairs, listed);
        } else {
#pragma unroll
            for (int k = 0; k < 2 * K; ++k) listed[k] = t.has(nbr[2 * half + k / K][k % K]);
        }
        int cnt = 0;
#pragma unroll
        for (int q = 2 * half; q < 2 * half + 2; ++q)
#pragma unroll
            for (int k = 0; k < K; ++k) {
                uint32_t v;
                if constexpr (SMALL_IDS)
                    v = (k & 1) ? nbr[q][k / 2] >> 16 : nbr[q][k / 2] & 0xFFFFu;
                else
                    v = nbr[q][k];
                const bool fresh = nb_ok[q] & (v < n) & !listed[(q - 2 * half) * K + k];
                queue[cnt][lane] = (QueueId<SMALL_IDS>)v;
                cnt += fresh ? 1 : 0;
            }
        // score the queued ids, QBATCH at a time, against the current 8th
        // entry; ids that beat it move with their logits to the front of the
        // column (the write index ns never passes the position just read).
        // The last batch may reach past the column's QCAP rows (QBATCH need
        // not divide QCAP): its rows are clamped for the read (the value is
        // then not used) and its slots past cnt write nothing, so that a
        // column whose every id passes is not written past its end.
        // Each batch is first screened (may_rank_before); the exact logits
        // are evaluated only when some lane holds an id the screen lets pass.
        const float ts = t.s[K - 1];
        const uint32_t ti = t.id[K - 1];
        int ns = 0;
        for (int it = 0; __any(it < cnt); it += QBATCH) {  // it is uniform
            uint32_t v[QBATCH];
#pragma unroll
            for (int b = 0; b < QBATCH; ++b)
                v[b] = (it + b < cnt) ? (uint32_t)queue[min(it + b, QCAP - 1)][lane] : EMPTY;
            Geo qg[QBATCH];
#pragma unroll
            for (int b = 0; b < QBATCH; ++b) qg[b] = load_geo_clamped(a.derived, n, v[b]);
            bool maybe[QBATCH], any_maybe = false;
#pragma unroll
            for (int b = 0; b < QBATCH; ++b) {
                maybe[b] = (it + b < cnt) & may_rank_before(qg[b], px, py, ts);  // queued ids are < n
                any_maybe |= maybe[b];
            }
            if (__any(any_maybe)) {
#pragma unroll
                for (int b = 0; b < QBATCH; ++b) {
                    const float sc = usable_logit(qg[b], v[b] < n, px, py);
                    const bool pass = maybe[b] & (sc == sc) & ranks_before(sc, v[b], ts, ti);  // false past cnt
                    if (it + b < cnt) {  // then ns <= it + b < cnt <= QCAP
                        queue[ns][lane] = (QueueId<SMALL_IDS>)v[b];  // a passing id is < n
                        qscore[ns][lane] = sc;
                    }
                    ns += pass ? 1 : 0;
                }
            }
        }
        // insert the survivors
        materialize(ns > 0);
        for (int u = 0; __any(u < ns); ++u) {
            const bool live = u < ns;
            const uint32_t v = live ? (uint32_t)queue[u][lane] : EMPTY;
            const float sc = live ? qscore[u][lane] : 0.0f;
            t.insert_if(sc, v, live);
        }
    }

    // 3. the tile's probe ids, culled by the tile bound
    if (a.inject > 0) {
        const float bx0 = (float)(tx * TILE) + 0.5f, by0 = (float)(ty * TILE) + 0.5f;
        const float bx1 = (float)min(tx * TILE + TILE - 1, a.w - 1) + 0.5f;
        const float by1 = (float)min(ty * TILE + TILE - 1, a.h - 1) + 0.5f;
        const float thr = wave_min(inside ? t.s[K - 1] : __builtin_inff());
        Geo pg;
        pg.g0 = make_float4(-1.f, -1.f, 0.f, 0.f);
        pg.g1 = make_float4(0.f, 0.f, 0.f, 0.f);
        uint64_t mask;
        if (a.probe_prev) {  // uniform
            // cull on the 16-byte records; the survivors' lanes then fetch their full records at once
            float4 pr = make_float4(-1.f, -1.f, 0.f, 0.f);
            if (lane < a.inject) pr = a.probe_prev[pid];
            const bool keep = (pr.x >= 0.0f) && probe_record_may_enter(pr, thr, bx0, bx1, by0, by1);
            if (keep) pg = load_geo(a.derived, pid);
            mask = __ballot(keep);
        } else {
            if (lane < a.inject) pg = load_geo(a.derived, pid);
            mask = __ballot((pg.g0.x >= 0.0f) && probe_may_enter(pg, thr, bx0, bx1, by0, by1));
        }
        while (mask) {
            // the survivor's record is in lane q's registers: broadcast it
            const int q = __builtin_ctzll(mask);
            mask &= mask - 1;
            const uint32_t id = (uint32_t)__builtin_amdgcn_readlane((int)pid, q);
            Geo g;
            g.g0.x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg.g0.x), q));
            g.g0.y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg.g0.y), q));
            g.g0.z = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg.g0.z), q));
            g.g0.w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg.g0.w), q));
            g.g1.x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg.g1.x), q));
            g.g1.y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg.g1.y), q));
            g.g1.z = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg.g1.z), q));
            g.g1.w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg.g1.w), q));
            const float s = logit(g, px, py);  // a survivor is an active site (checked above)
            const bool ok = inside & (s == s);
            // a candidate that does not rank before the 8th entry leaves the list as it is
            const bool beats = ok & ranks_before(s, id, t.s[K - 1], t.id[K - 1]);
            if (__any(beats)) {
                materialize(beats);
                t.insert_if(s, id, beats);
            }
        }
    }

    if (inside) {
        if constexpr (NEXT16) {
            // ids < n <= 0xFFFF keep their value; EMPTY saturates to 0xffff
            *reinterpret_cast<uint4*>(a.next16 + ((size_t)j * a.w + i) * K) =
                make_uint4(pack16(t.id[0], t.id[1]), pack16(t.id[2], t.id[3]), pack16(t.id[4], t.id[5]),
                           pack16(t.id[6], t.id[7]));
        } else {
            uint4* o = reinterpret_cast<uint4*>(a.next + ((size_t)j * a.w + i) * K);
            o[0] = make_uint4(t.id[0], t.id[1], t.id[2], t.id[3]);
            o[1] = make_uint4(t.id[4], t.id[5], t.id[6], t.id[7]);
        }
        if (a.next_thr) a.next_thr[(size_t)j * a.w + i] = t.s[K - 1];
    }
    if (a.next_scores) materialize(true);  // uniform; a no-op unless THR_IN
    if (inside) {
        if (a.next_scores) {
            float4* os = reinterpret_cast<float4*>(a.next_scores + ((size_t)j * a.w + i) * K);
            os[0] = make_float4(t.s[0], t.s[1], t.s[2], t.s[3]);
            os[1] = make_float4(t.s[4], t.s[5], t.s[6], t.s[7]);
        }
    }
    if (lazy_out) *lazy_out = lazy;
}

// Argument checks of a propagation pass (shared by the entry points that run
// one) and its kernel arguments.  Returns SAD_OK with a filled in, or the
// error status.
inline int prop_setup(const float* derived, int32_t n, int32_t h, int32_t w, const sad_pass_maps& m, int32_t stride,
                      uint64_t seed, uint32_t pass_index, int32_t inject_per_tile, PropArgs& a) {
    if (!sites_ok(n) || !image_ok(h, w) || stride < 1 || inject_per_tile < 0) return SAD_EINVAL;
    if ((m.prev_bits != 16 && m.prev_bits != 32) || (m.next_bits != 16 && m.next_bits != 32)) return SAD_EINVAL;
    if (inject_per_tile > SAD_MAX_INJECT) return SAD_EUNSUPPORTED;
    // a 16-bit map needs every usable id below 0xffff, its empty slot
    if ((m.prev_bits == 16 || m.next_bits == 16) && n > SMALL_IDS_MAX) return SAD_EUNSUPPORTED;
    const int64_t pix = int64_t(h) * w;
    const int64_t pbytes = pix * K * (m.prev_bits / 8), nbytes = pix * K * (m.next_bits / 8), sbytes = pix * K * 4;
    const int64_t tbytes = pix * 4, rbytes = int64_t(n) * 16, dbytes = int64_t(n) * REC * 4;
    if (!array_ok(derived, n, 16) || !array_ok(m.topk_next, pix, 16)) return SAD_EINVAL;
    if ((m.topk_prev && !aligned(m.topk_prev, 16)) || (m.scores_prev && !aligned(m.scores_prev, 16)) ||
        (m.scores_next && !aligned(m.scores_next, 16)) || (m.probe_prev && !aligned(m.probe_prev, 16)) ||
        (m.probe_next && !aligned(m.probe_next, 16)))
        return SAD_EINVAL;
    if ((m.scores_prev || m.thr_prev) && !m.topk_prev) return SAD_EINVAL;
    if (m.scores_prev && m.thr_prev) return SAD_EINVAL;
    if ((m.thr_prev && !aligned(m.thr_prev, 4)) || (m.thr_next && !aligned(m.thr_next, 4))) return SAD_EINVAL;
    // no two buffers may share memory
    const void* outs[4] = {m.topk_next, m.scores_next, m.thr_next, m.probe_next};
    const int64_t obytes[4] = {nbytes, sbytes, tbytes, rbytes};
    const void* ins[5] = {m.topk_prev, m.scores_prev, m.thr_prev, m.probe_prev, derived};
    const int64_t ibytes[5] = {pbytes, sbytes, tbytes, rbytes, dbytes};
    for (int o = 0; o < 4; ++o) {
        for (int q = 0; q < 5; ++q)
            if (overlap(outs[o], obytes[o], ins[q], ibytes[q])) return SAD_EINVAL;
        for (int q = o + 1; q < 4; ++q)
            if (overlap(outs[o], obytes[o], outs[q], obytes[q])) return SAD_EINVAL;
    }
    for (int o = 0; o < 5; ++o)
        for (int q = o + 1; q < 5; ++q)
            if (overlap(ins[o], ibytes[o], ins[q], ibytes[q])) return SAD_EINVAL;
    const int64_t ntiles = int64_t(tiles_x(w)) * tiles_y(h);
    if (ntiles > MAX_TILES) return SAD_EINVAL;
    a.derived = derived;
    a.prev = m.prev_bits == 32 ? static_cast<const uint32_t*>(m.topk_prev) : nullptr;
    a.prev16 = m.prev_bits == 16 ? static_cast<const uint16_t*>(m.topk_prev) : nullptr;
    a.prev_scores = m.scores_prev;
    a.prev_thr = m.thr_prev;
    a.next = m.next_bits == 32 ? static_cast<uint32_t*>(m.topk_next) : nullptr;
    a.next16 = m.next_bits == 16 ? static_cast<uint16_t*>(m.topk_next) : nullptr;
    a.next_scores = m.scores_next;
    a.next_thr = m.thr_next;
    a.probe_prev = reinterpret_cast<const float4*>(m.probe_prev);
    a.probe_next = reinterpret_cast<float4*>(m.probe_next);
    a.seed = seed;
    a.n = n;
    a.h = h;
    a.w = w;
    a.stride = stride;
    a.inject = n > 0 ? inject_per_tile : 0;
    a.tiles_x = tiles_x(w);
    a.n_tiles = (int32_t)ntiles;
    a.pass_index = pass_index;
    return SAD_OK;
}

// The maps of sad_propagate_topk and sad_step_fused in a sad_pass_maps.
inline sad_pass_maps maps32(const uint32_t* topk_prev, const float* scores_prev, uint32_t* topk_next,
                            float* scores_next) {
    sad_pass_maps m = {};
    m.topk_prev = topk_prev;
    m.prev_bits = 32;
    m.scores_prev = scores_prev;
    m.topk_next = topk_next;
    m.next_bits = 32;
    m.scores_next = scores_next;
    return m;
}

}  // namespace sad
