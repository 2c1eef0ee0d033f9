// sad_backward.hip -- the loss and the hand-derived gradients of the soft
// anisotropic render (Sec. 6.1 loss; Appendix B.4 "Per-pixel gradients"),
// summed per site on chip before they leave the workgroup (Sec. 4.8
// "Gradient Accumulation"), and the call that runs a propagation pass and
// the backward over its lists.
//
// One workgroup per region of 32 x 16 pixels (sad_region.h), in two phases:
//
//  A. Pixel-major, one lane per pixel.  Every listed site claims a slot of
//     the region's LDS table and counts its entry there; the claimed sites'
//     records are read once into LDS; the counts become bucket starts and
//     the buckets are cut into pieces of at most PIECE entries.  The pixel's
//     forward follows: float32 logits (the ranking's own values), their
//     exponentials, and then in float64 the normaliser, the blended colour,
//     the residual and dL/dc.  What the second phase needs of the pixel
//     (the largest logit, 1/Z, dL/dc and dL/dc . c) goes to LDS, and the
//     pixel's index goes to the bucket of each of its entries: a counting
//     sort of the region's entries by site.
//  B. Site-major, one piece per lane.  A lane holds one site's record and
//     runs over the piece's pixels, recomputing each entry's logit and weight
//     from the pixel's values, forming the 10 terms of Appendix B.4 in
//     float64 and summing them in registers; the piece's sums are then added
//     to the slot's float64 sums in LDS (one LDS add per term per piece,
//     rather than one per term per list entry).
// Finally every slot's 10 sums leave the workgroup as float atomics on the
// site's gradient record, once per (region, site).
//
// Precision: the residual c - I and the differences c_i - c cancel when the
// render is close to the target or the site's colour to the blend; carried
// in float64 they leave the gradients within a few float32 roundings of the
// exact sums (the per-entry float32 inputs are the logits, the hardware
// exponential of l - max l and the reciprocal square root of q).
#include "sad_propagate.h"
#include "sad_region.h"

namespace sad {

constexpr int PIECE = 10;  // entries of one site per phase-B lane
// The per-slot sums are term-major with a row of SLOTS + 1 doubles: the
// lanes of one phase-B add (different slots, one term) and of one phase-C
// read (one slot, different terms) fall in different LDS banks.
constexpr int ACC_ROW = SLOTS + 1;
// at most ceil(cnt / PIECE) pieces per slot: sum over slots <= entries / PIECE + SLOTS
constexpr int MAX_PIECES = REGION_PIX * K / PIECE + SLOTS;
constexpr int BWD_THREADS = WAVE * REGION_WAVES;
constexpr int SLOT_WAVES = SLOTS / WAVE;  // wavefronts that plan the buckets, one slot per lane
static_assert(SLOTS % WAVE == 0 && SLOT_WAVES <= REGION_WAVES, "slot planning layout");
static_assert(SLOTS <= 256, "slots are packed in 8 bits");

struct BwdArgs {
    const float* derived;
    const uint32_t* topk;
    const float* target;
    float* grad;
    float* loss;
    float* image;
    int32_t n, h, w;
    RegionGrid rg;
    double inv_p;  // 1 / (h w)
};

// Site values for the gradient terms, in float64: geometry, and
// (1/s1^2 - 1/s2^2) formed without cancellation.
struct SiteD {
    double x, y, tau, cs, sn, is1, is2, dsq;
};

__device__ __forceinline__ SiteD site_d(float4 g0, float4 g1) {
    const double is1 = (double)g1.z, is2 = (double)g1.w;
    return {(double)g0.x, (double)g0.y, (double)g0.z, (double)g1.x, (double)g1.y, is1, is2, (is1 - is2) * (is1 + is2)};
}

// Add the 10 terms of one list entry (Appendix B.4) to sum, in the gradient
// record's order (x, y, log tau, r, colour, theta, log s1, log s2): (px, py)
// the pixel centre, l the entry's float32 logit, w its weight, delta = dL/dl
// = w (g.c_i - g.c) and g = dL/dc.  With a_r = dx cos + dy sin, b_r = dy cos
// - dx sin, a = a_r/s1, b = b_r/s2, q = a^2 + b^2 and u = tau delta / sqrt(q)
// (= -2 kappa): x: u (a cos/s1 - b sin/s2), y: u (a sin/s1 + b cos/s2),
// theta: -u a_r b_r (1/s1^2 - 1/s2^2), log s1: u a^2, log s2: u b^2; at q = 0
// (the pixel centre on the site) u is taken as 0.  Written with shared
// factors and fused multiply-adds, all in float64.
__device__ __forceinline__ void add_entry_terms(const SiteD& s, double px, double py, float l, double w,
                                                double delta, const double (&g)[3], double (&sum)[NGRAD]) {
    sum[4] = fma(w, g[0], sum[4]);
    sum[5] = fma(w, g[1], sum[5]);
    sum[6] = fma(w, g[2], sum[6]);
    sum[2] = fma(delta, (double)l, sum[2]);
    sum[3] = fma(s.tau, delta, sum[3]);
    const double dx = px - s.x, dy = py - s.y;
    const double ar = fma(dx, s.cs, dy * s.sn), br = fma(dy, s.cs, -(dx * s.sn));
    const double a = ar * s.is1, b = br * s.is2;
    const double q = fma(a, a, b * b);
    // 1/sqrt(q): the hardware estimate refined by one Newton step
    const double r0 = __builtin_amdgcn_rsq(q);
    const double rs = q > 0.0 ? r0 * fma(-0.5 * q, r0 * r0, 1.5) : 0.0;
    const double u = s.tau * delta * rs;
    const double ua = u * a, ub = u * b;
    const double A = ua * s.is1, B = ub * s.is2;
    sum[0] = fma(A, s.cs, fma(-B, s.sn, sum[0]));
    sum[1] = fma(A, s.sn, fma(B, s.cs, sum[1]));
    sum[7] = fma(-(u * s.dsq), ar * br, sum[7]);
    sum[8] = fma(ua, a, sum[8]);
    sum[9] = fma(ub, b, sum[9]);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
}

// A lane's slot and position in the slot's bucket for list entry k, packed as
// slot | position << 8 (NOSLOT when the entry has no slot).
constexpr uint32_t NOSLOT = 0xFFFFFFFFu;

// Claim a slot of the region's table for every id < n of the lane's list
// (the probing of claim_slots): slot16[k / 2] holds entry k's slot in its
// k-th 16-bit half, 0xFFFF when the entry has no slot.  Branch-free: every
// round reads the probed slot of all 8 entries (a read of one address by many
// lanes is a broadcast), and compare-and-swaps only where a lane saw an
// empty slot; the other lanes of that instruction aim it at their own word of
// `mine` (which never holds EMPTY), so the instruction neither branches nor
// touches the table for them.
__device__ __forceinline__ void claim(uint32_t* keys, uint32_t* mine, const uint32_t (&ids)[K], uint32_t n,
                                      uint32_t (&slot16)[K / 2]) {
    uint32_t pos[K], pend = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        pos[k] = slot_hash(ids[k]);
        pend |= (ids[k] < n ? 1u : 0u) << k;
    }
    for (int round = 0; round < REGION_PROBES && __any(pend != 0); ++round) {
        uint32_t cur[K];
#pragma unroll
        for (int k = 0; k < K; ++k) cur[k] = keys[pos[k]];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const bool take = ((pend >> k) & 1) && cur[k] == EMPTY;
            const uint32_t got = atomicCAS(take ? &keys[pos[k]] : mine, EMPTY, ids[k]);
            cur[k] = take ? got : cur[k];
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const bool live = (pend >> k) & 1;
            const bool hit = (cur[k] == EMPTY) | (cur[k] == ids[k]);  // claimed now, or before
            pend &= ~((live && hit ? 1u : 0u) << k);
            pos[k] = live && !hit ? (pos[k] + slot_step(ids[k])) & (SLOTS - 1) : pos[k];
        }
    }
#pragma unroll
    for (int k = 0; k < K; k += 2) {
        const uint32_t s0 = (ids[k] < n && !((pend >> k) & 1)) ? pos[k] : 0xFFFFu;
        const uint32_t s1 = (ids[k + 1] < n && !((pend >> (k + 1)) & 1)) ? pos[k + 1] : 0xFFFFu;
        slot16[k / 2] = s0 | (s1 << 16);
    }
}

__device__ __forceinline__ int slot_of(const uint32_t (&slot16)[K / 2], int k) {
    const uint32_t v = (k & 1) ? slot16[k / 2] >> 16 : slot16[k / 2] & 0xFFFFu;
    return v == 0xFFFFu ? -1 : (int)v;
}

// What phase B needs of a pixel, in one 32-byte record (two 16-byte LDS
// reads): the largest logit, dL/dc (float32, formed in float64), 1/Z and
// dL/dc . c (float64, c the blended colour).
struct __attribute__((aligned(16))) PixState {
    float m, g0, g1, g2;
    double iz, gc;
};

// With n <= SMALL_IDS_MAX sites, slots are the ranks of the region's listed
// ids (claim_ranked) from a bitmap of RANK_WORDS words.
constexpr int RANK_WORDS = (SMALL_IDS_MAX + 1) / 32;
static_assert(RANK_WORDS == 4 * BWD_THREADS, "each thread ranks four bitmap words");

// The backward's LDS.
struct BwdLds {
    uint32_t keys[SLOTS];
    uint32_t cnt[SLOTS];            // entries per slot
    uint32_t bstart[SLOTS];         // the slot's first position in `order`
    uint32_t pstart[SLOTS];         // the slot's first piece
    uint8_t piece_slot[(MAX_PIECES + 15) / 16 * 16];  // each piece's slot
    uint32_t wtot[SLOT_WAVES][2];   // entries and pieces of each planning wavefront's slots
    uint32_t mine[BWD_THREADS];     // one word per lane that never holds EMPTY (see claim)
    uint32_t wscan[REGION_WAVES];   // per-wavefront totals of the rank scan (claim_ranked)
    union {
        struct {
            uint16_t order[REGION_PIX * K];  // pixels of the region's entries, grouped by slot
            PixState ps[REGION_PIX];         // what phase B needs of each pixel
        } ph;
        struct {                                // during claim_ranked only
            uint32_t bits[RANK_WORDS];          // one bit per site id listed in the region
            uint16_t rank[RANK_WORDS];          // listed sites below each word's first id
        } cl;
    } x;
    // the claimed sites' records during the forward, then the per-slot sums
    // of phase B
    __attribute__((aligned(16))) double shared_sums[NGRAD * ACC_ROW];
    double wsum[REGION_WAVES];
    uint32_t npieces;
};
static_assert(sizeof(float4) * 3 * SLOTS <= sizeof(double) * NGRAD * ACC_ROW, "records fit where the sums go");

// The slots of the lane's entries when every id fits the bitmap (n <=
// SMALL_IDS_MAX): every listed id sets its bit (one OR per entry, no retries),
// a prefix count over the bitmap gives each id its rank among the region's
// distinct listed ids, and that rank is its slot; ids ranked SLOTS or later
// get none (0xFFFF, as in claim).  The bitmap must be zero and a barrier
// passed before the call; ends with the slots' keys written but not yet
// visible to other wavefronts (the caller's barrier follows).
__device__ __forceinline__ void claim_ranked(BwdLds& L, const uint32_t (&ids)[K], uint32_t n,
                                             uint32_t (&slot16)[K / 2]) {
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
#pragma unroll
    for (int k = 0; k < K; ++k)
        if (ids[k] < n) atomicOr(&L.x.cl.bits[ids[k] >> 5], 1u << (ids[k] & 31));
    __syncthreads();
    // thread t ranks words 4t .. 4t + 3: an exclusive prefix of the set bits
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        c[j] = __builtin_popcount(L.x.cl.bits[4 * tid + j]);
        tot += c[j];
    }
    uint32_t inc = tot;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t u = __shfl_up(inc, off, WAVE);
        if (lane >= off) inc += u;
    }
    if (lane == WAVE - 1) L.wscan[wv] = inc;
    __syncthreads();
    uint32_t base = inc - tot;
#pragma unroll
    for (int w2 = 0; w2 < REGION_WAVES; ++w2) base += w2 < wv ? L.wscan[w2] : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        L.x.cl.rank[4 * tid + j] = (uint16_t)base;  // <= REGION_PIX * K
        base += c[j];
    }
    __syncthreads();
    uint32_t sl[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        sl[k] = 0xFFFFu;
        if (ids[k] < n) {
            const uint32_t w = ids[k] >> 5;
            const uint32_t r = L.x.cl.rank[w] + __builtin_popcount(L.x.cl.bits[w] & ((1u << (ids[k] & 31)) - 1u));
            if (r < (uint32_t)SLOTS) {
                sl[k] = r;
                L.keys[r] = ids[k];  // every lane listing the id writes the same value
            }
        }
    }
#pragma unroll
    for (int k = 0; k < K; k += 2) slot16[k / 2] = sl[k] | (sl[k + 1] << 16);
}

// The tables of the region cleared (call on every thread, then a barrier).
__device__ __forceinline__ void clear_tables(BwdLds& L, uint32_t n) {
    const int tid = threadIdx.x;
    for (int s = tid; s < SLOTS; s += BWD_THREADS) {
        L.keys[s] = EMPTY;
        L.cnt[s] = 0;
    }
    L.mine[tid] = 0;
    if (n <= (uint32_t)SMALL_IDS_MAX)  // uniform
#pragma unroll
        for (int j = 0; j < 4; ++j) L.x.cl.bits[4 * tid + j] = 0u;
}

// Rotate the lane's 8 entries left by (lane + lane / 8) mod 8 (anti-diagonal
// of the tile), so that neighbouring pixels listing the same site at the same
// rank claim and count it in different instructions (same-address LDS atomics
// of one instruction are serialised).  Three selects per entry; the empty asm
// after each stage keeps the compiler from merging the stages into an 8-way
// select per entry.
template <class T>
struct Row8 {
    T v[K];
};

template <class T>
__device__ __forceinline__ Row8<T> rotate_lane(Row8<T> r, int lane) {
    const int rot = (lane + (lane >> 3)) & (K - 1);
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
        const bool on = (rot >> bit) & 1;
        T u[K];
#pragma unroll
        for (int k = 0; k < K; ++k) u[k] = on ? r.v[(k + (1 << bit)) & (K - 1)] : r.v[k];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            r.v[k] = u[k];
            asm volatile("" : "+v"(r.v[k]));
        }
    }
    return r;
}

// The backward of one region, from each lane's list (ids, in any order) and
// target colour; with GIVEN_LOGITS, given[k] is entry k's float32 logit at
// the pixel (as the propagation pass computed it) and the forward does not
// evaluate it again.  The tables of L must be cleared (clear_tables) and a
// barrier passed before the call.
template <bool GIVEN_LOGITS>
__device__ __forceinline__ void backward_region(const BwdArgs& a, BwdLds& L, int rx, int ry, uint32_t (&ids)[K],
                                                const float (&given)[K], const float (&tg)[3]) {
    const uint32_t n = (uint32_t)a.n;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    int i, j;
    region_pixel(rx, ry, wv, lane, i, j);
    const bool inside = i < a.w && j < a.h;
    const size_t p = (size_t)j * a.w + i;
    const float px = (float)i + 0.5f, py = (float)j + 0.5f;
    float4* recs = reinterpret_cast<float4*>(L.shared_sums);  // [SLOTS][3]
    double* acc = L.shared_sums;                              // [NGRAD][ACC_ROW]

    // A1. a slot for every listed site
    uint32_t slot16[K / 2];
    if (n <= (uint32_t)SMALL_IDS_MAX)  // uniform
        claim_ranked(L, ids, n, slot16);
    else
        claim(L.keys, &L.mine[tid], ids, n, slot16);
    __syncthreads();

    // A2. every claimed site's record is read from memory once, into LDS
    for (int s = tid; s < SLOTS; s += BWD_THREADS) {
        const uint32_t id = L.keys[s];
        if (id == EMPTY) continue;
        const float4* r = reinterpret_cast<const float4*>(a.derived + (size_t)id * REC);
        recs[s * 3 + 0] = r[0];
        recs[s * 3 + 1] = r[1];
        recs[s * 3 + 2] = r[2];
    }
    __syncthreads();

    // A3. the pixel's forward: float32 logits, their exponentials, then in
    //     float64 the normaliser, the blend, the residual and dL/dc.  When an
    //     entry of some lane of the wavefront found no slot, the wavefront
    //     takes a copy of this code that reads such records from memory;
    //     otherwise every record read is an LDS read (one pointer that may
    //     point to either memory would make every read a slower generic load).
    bool slotted = true;
#pragma unroll
    for (int k = 0; k < K; ++k) slotted &= (ids[k] >= n) | (slot_of(slot16, k) >= 0);
    double lsum = 0.0;
    auto forward = [&](auto lds_only) {
        // part q (0: x y tau r, 1: cos sin 1/s1 1/s2, 2: colour) of entry k's record
        auto rec = [&](int k, int q) -> float4 {
            const int sk = slot_of(slot16, k);
            if constexpr (decltype(lds_only)::value)
                return recs[(sk >= 0 ? sk : 0) * 3 + q];
            else
                return sk >= 0 ? recs[sk * 3 + q] : reinterpret_cast<const float4*>(a.derived + (size_t)ids[k] * REC)[q];
        };
        float l[K], e[K];
        float mx = -__builtin_inff();
#pragma unroll
        for (int k = 0; k < K; ++k) {
            l[k] = __builtin_nanf("");
            if (ids[k] >= n) continue;
            float s;
            if constexpr (GIVEN_LOGITS) {
                s = given[k];  // the pass's own float32 logit of the entry
            } else {
                Geo g;
                g.g0 = rec(k, 0);
                g.g1 = rec(k, 1);
                s = usable_logit(g, true, px, py);
            }
            if (!finitef(s)) continue;
            l[k] = s;
            mx = fmaxf(mx, s);
        }
        double z = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            e[k] = finitef(l[k]) ? __expf(l[k] - mx) : 0.0f;
            z += (double)e[k];
        }
        const double iz = z > 0.0 ? 1.0 / z : 0.0;
        double c[3] = {0.0, 0.0, 0.0};
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (!finitef(l[k])) continue;
            const double wk = (double)e[k] * iz;
            const float4 col = rec(k, 2);
            c[0] = fma(wk, (double)col.x, c[0]);
            c[1] = fma(wk, (double)col.y, c[1]);
            c[2] = fma(wk, (double)col.z, c[2]);
        }
        float g[3];
        double gc = 0.0;
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
            const double r = c[ch] - (double)tg[ch];
            lsum = fma(r, r, lsum);
            g[ch] = (float)(2.0 * r * a.inv_p);
            gc = fma((double)g[ch], c[ch], gc);
        }
        if (inside && a.image) {
            a.image[p * 3 + 0] = (float)c[0];
            a.image[p * 3 + 1] = (float)c[1];
            a.image[p * 3 + 2] = (float)c[2];
        }
        PixState st;
        st.m = mx == -__builtin_inff() ? 0.0f : mx;
        st.g0 = g[0];
        st.g1 = g[1];
        st.g2 = g[2];
        st.iz = iz;
        st.gc = gc;
        L.x.ph.ps[tid] = st;
    };
    if (__all(slotted))
        forward(std::true_type{});
    else
        forward(std::false_type{});
    if (a.loss) {
        const double ws = wave_sum_d(lsum);
        if (lane == 0) L.wsum[wv] = ws;
    }
    // each entry's position in its slot's bucket (slots without a site
    // count in the lane's own word)
    uint32_t sp[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int sk = slot_of(slot16, k);
        const uint32_t c = atomicAdd(sk >= 0 ? &L.cnt[sk] : &L.mine[tid], 1u);
        sp[k] = sk >= 0 ? (uint32_t)sk | (c << 8) : NOSLOT;
    }
    __syncthreads();  // counts complete; records no longer read

    // A4. buckets and pieces: each of the first SLOT_WAVES wavefronts scans
    //     the entry counts of its slots (one per lane) and their piece counts
    //     (ceil(count / PIECE)); the others clear the per-slot sums (where
    //     the records were)
    uint32_t my_c = 0, my_pc = 0, ex_c = 0, ex_pc = 0;
    if (wv < SLOT_WAVES) {
        my_c = L.cnt[tid];
        my_pc = (my_c + PIECE - 1) / PIECE;
        uint32_t ic = my_c, ip = my_pc;  // inclusive scans over the wavefront
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const uint32_t u = __shfl_up(ic, off, WAVE), v = __shfl_up(ip, off, WAVE);
            if (lane >= off) {
                ic += u;
                ip += v;
            }
        }
        ex_c = ic - my_c;
        ex_pc = ip - my_pc;
        if (lane == WAVE - 1) {
            L.wtot[wv][0] = ic;
            L.wtot[wv][1] = ip;
        }
    } else {
        for (int s = tid - SLOT_WAVES * WAVE; s < NGRAD * ACC_ROW; s += BWD_THREADS - SLOT_WAVES * WAVE) acc[s] = 0.0;
    }
    __syncthreads();  // wavefront totals
    if (wv < SLOT_WAVES) {
        uint32_t bc = 0, bp = 0, tc = 0, tp = 0;
#pragma unroll
        for (int w2 = 0; w2 < SLOT_WAVES; ++w2) {
            bc += w2 < wv ? L.wtot[w2][0] : 0u;
            bp += w2 < wv ? L.wtot[w2][1] : 0u;
            tp += L.wtot[w2][1];
            tc += L.wtot[w2][0];
        }
        L.bstart[tid] = bc + ex_c;
        L.pstart[tid] = bp + ex_pc;
        for (uint32_t k = 0; k < my_pc; ++k) L.piece_slot[bp + ex_pc + k] = (uint8_t)tid;  // tid < SLOTS
        if (tid == 0) L.npieces = tp;
        (void)tc;
    }
    __syncthreads();  // buckets planned

    // A5. counting sort: the pixel's index into the bucket of each entry.
    //     Entries without a slot (the region lists more sites than its table
    //     holds; rare) send their terms to memory directly.
    uint32_t lone = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (sp[k] != NOSLOT)
            L.x.ph.order[L.bstart[sp[k] & 0xFFu] + (sp[k] >> 8)] = (uint16_t)tid;
        else if (ids[k] < n)
            lone |= 1u << k;
    }
    if (lone) {
        const PixState st = L.x.ph.ps[tid];
        const double g[3] = {(double)st.g0, (double)st.g1, (double)st.g2};
        for (; lone; lone &= lone - 1) {
            const int k = __builtin_ctz(lone);
            uint32_t id = ids[0];
#pragma unroll
            for (int kk = 1; kk < K; ++kk) id = k == kk ? ids[kk] : id;
            const Geo gk = load_geo(a.derived, id);
            const float l = usable_logit(gk, true, px, py);
            if (!finitef(l)) continue;
            const float4 col = reinterpret_cast<const float4*>(a.derived + (size_t)id * REC)[2];
            const double wk = (double)__expf(l - st.m) * st.iz;
            const double delta =
                wk * (fma(g[0], (double)col.x, fma(g[1], (double)col.y, g[2] * (double)col.z)) - st.gc);
            double t[NGRAD];
#pragma unroll
            for (int q = 0; q < NGRAD; ++q) t[q] = 0.0;
            add_entry_terms(site_d(gk.g0, gk.g1), (double)px, (double)py, l, wk, delta, g, t);
#pragma unroll
            for (int q = 0; q < NGRAD; ++q) unsafeAtomicAdd(&a.grad[(size_t)id * REC + q], (float)t[q]);
        }
    }
    __syncthreads();

    // B. one piece per lane: a site's entries, pieces dealt across the
    //    wavefronts in turn
    const uint32_t np = L.npieces;
    for (uint32_t base = 0; base < np; base += BWD_THREADS) {
        const uint32_t pc = base + (uint32_t)(lane * REGION_WAVES + wv);
        if (pc >= np) continue;
        const int s = L.piece_slot[pc];
        const uint32_t kp = pc - L.pstart[s];
        const int start = (int)(L.bstart[s] + kp * PIECE);
        const int len = (int)min((uint32_t)PIECE, L.cnt[s] - kp * PIECE);
        const uint32_t id = L.keys[s];
        const Geo geo = load_geo(a.derived, id);
        const float4 col = reinterpret_cast<const float4*>(a.derived + (size_t)id * REC)[2];
        const SiteD sd = site_d(geo.g0, geo.g1);
        const double cr = (double)col.x, cg = (double)col.y, cb = (double)col.z;
        const bool active = geo.g0.x >= 0.0f;  // a claimed id is < n; an inactive site has x < 0
        double sum[NGRAD];
#pragma unroll
        for (int q = 0; q < NGRAD; ++q) sum[q] = 0.0;
        // the next entry's pixel is read one trip ahead (len >= 1)
        const int last = start + len - 1;
        int pp = L.x.ph.order[start];
        for (int it = 0; it < len; ++it) {
            const PixState st = L.x.ph.ps[pp];
            const int pp_next = L.x.ph.order[min(start + it + 1, last)];
            int pi, pj;
            region_pixel(rx, ry, pp / WAVE, pp & (WAVE - 1), pi, pj);
            const float fx = (float)pi + 0.5f, fy = (float)pj + 0.5f;
            const float l = logit(geo, fx, fy);
            // unusable entries take no part (as in the forward)
            if (active & finitef(l)) {
                const double wk = (double)__expf(l - st.m) * st.iz;
                const double g[3] = {(double)st.g0, (double)st.g1, (double)st.g2};
                const double delta = wk * (fma(g[0], cr, fma(g[1], cg, g[2] * cb)) - st.gc);
                add_entry_terms(sd, (double)fx, (double)fy, l, wk, delta, g, sum);
            }
            pp = pp_next;
        }
#pragma unroll
        for (int q = 0; q < NGRAD; ++q) atomicAdd(&acc[q * ACC_ROW + s], sum[q]);
    }
    __syncthreads();

    // C. the region's per-site sums leave the workgroup: one float atomic per
    //    (site, term), a site's 10 terms from consecutive lanes (one or two
    //    cache lines per site instead of one per lane)
    for (int pr = tid; pr < NGRAD * SLOTS; pr += BWD_THREADS) {
        const int s = pr / NGRAD, q = pr % NGRAD;
        const uint32_t id = L.keys[s];
        if (id == EMPTY) continue;
        const double v = acc[q * ACC_ROW + s];
        if (v != 0.0) unsafeAtomicAdd(&a.grad[(size_t)id * REC + q], (float)v);
    }
    if (a.loss && tid == 0) {
        double tot = 0.0;
        for (int k = 0; k < REGION_WAVES; ++k) tot += L.wsum[k];
        unsafeAtomicAdd(a.loss, (float)(tot * a.inv_p));
    }
}

__global__ __launch_bounds__(BWD_THREADS) __attribute__((amdgpu_waves_per_eu(6))) void k_backward(BwdArgs a) {
    __shared__ BwdLds L;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int reg = xcd_block(blockIdx.x, gridDim.x);
    const int rx = reg % a.rg.rgx, ry = reg / a.rg.rgx;
    int i, j;
    region_pixel(rx, ry, wv, lane, i, j);
    const bool inside = i < a.w && j < a.h;
    const size_t p = (size_t)j * a.w + i;

    clear_tables(L, (uint32_t)a.n);

    uint32_t ids[K];
    float tg[3] = {0.f, 0.f, 0.f};
    {
        uint4 l0 = make_uint4(EMPTY, EMPTY, EMPTY, EMPTY), l1 = l0;
        if (inside) {
            const uint4* l = reinterpret_cast<const uint4*>(a.topk + p * K);
            l0 = l[0];
            l1 = l[1];
            tg[0] = a.target[p * 3 + 0];
            tg[1] = a.target[p * 3 + 1];
            tg[2] = a.target[p * 3 + 2];
        }
        const Row8<uint32_t> r = rotate_lane(Row8<uint32_t>{{l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w}}, lane);
#pragma unroll
        for (int k = 0; k < K; ++k) ids[k] = r.v[k];
    }
    __syncthreads();  // table cleared
    const float none[K] = {};
    backward_region<false>(a, L, rx, ry, ids, none, tg);
}

// The propagation pass's LDS for the eight wavefronts of a region.
template <bool SMALL_IDS>
struct PassLds {
    QueueId<SMALL_IDS> queue[REGION_WAVES][QCAP][WAVE];
    float qscore[REGION_WAVES][QCAP][WAVE];
};

// A training iteration's last propagation pass and the backward over its
// lists in one kernel (Sec. 6.6 / Table 9 one-pass update, then Sec. 4.8 /
// Appendix B.4).  A workgroup takes one region: each wavefront runs the pass
// on its tile of the region (propagate_tile: the next lists, with 32-bit or
// 16-bit ids, and logits are written as by sad_propagate_pass), keeps the
// tile's new lists with their
// float32 logits in registers, and after a barrier the region's backward
// starts from them in the same LDS: no list is read back and no logit of the
// forward is evaluated again, and regions start their backward while others
// still run their pass.
template <bool SMALL_IDS, bool PREV16, bool THR_IN, bool NEXT16>
__global__ __launch_bounds__(BWD_THREADS) __attribute__((amdgpu_waves_per_eu(SMALL_IDS ? 6 : 1)))
void k_step_last(PropArgs pa, BwdArgs a) {
    __shared__ union {
        PassLds<SMALL_IDS> pass;
        BwdLds bwd;
    } lds;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int reg = xcd_block(blockIdx.x, gridDim.x);
    const int rx = reg % a.rg.rgx, ry = reg / a.rg.rgx;
    const int tx = rx * RT_X + wv % RT_X, ty = ry * RT_Y + wv / RT_X;
    TopK t;
    t.clear();
    if (tx < pa.tiles_x && ty * pa.tiles_x + tx < pa.n_tiles)  // uniform per wavefront
        propagate_tile<SMALL_IDS, PREV16, NEXT16, THR_IN>(pa, ty * pa.tiles_x + tx, lds.pass.queue[wv],
                                                         lds.pass.qscore[wv], t);
    int i, j;
    region_pixel(rx, ry, wv, lane, i, j);  // the pixel the pass just listed
    float tg[3] = {0.f, 0.f, 0.f};
    if (i < a.w && j < a.h) {
        const size_t p = (size_t)j * a.w + i;
        tg[0] = a.target[p * 3 + 0];
        tg[1] = a.target[p * 3 + 1];
        tg[2] = a.target[p * 3 + 2];
    }
    uint32_t ids[K];
    float lg[K];
    {
        Row8<uint32_t> ri;
        Row8<float> rl;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            ri.v[k] = t.id[k];
            rl.v[k] = t.s[k];
        }
        ri = rotate_lane(ri, lane);
        rl = rotate_lane(rl, lane);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            ids[k] = ri.v[k];
            lg[k] = rl.v[k];
        }
    }
    __syncthreads();  // the pass's queues are no longer read
    clear_tables(lds.bwd, (uint32_t)a.n);
    __syncthreads();  // table cleared
    // with only the 8th logits given (THR_IN) the lanes' other logits are not
    // all known: the forward evaluates them from the site records it stages
    // in LDS (the same float32 values)
    backward_region<!THR_IN>(a, lds.bwd, rx, ry, ids, lg, tg);
}

// Argument checks of a backward pass over the list map topk, and its kernel
// arguments.  Returns SAD_OK with b filled in, or the error status.
inline int bwd_setup(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                     const float* target, float* grad, float* loss, float* image, BwdArgs& b, int id_bits = 32) {
    if (!sites_ok(n) || !image_ok(h, w)) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(derived, n, 16) || !array_ok(topk, pix, 16)) return SAD_EINVAL;
    if (!array_ok(target, pix, 4) || !array_ok(grad, n, 16)) return SAD_EINVAL;
    if ((loss && !aligned(loss, 4)) || (image && !aligned(image, 4))) return SAD_EINVAL;
    // the outputs may overlap neither each other nor any input
    const int64_t gbytes = int64_t(n) * REC * 4;
    const void* outs[3] = {grad, loss, image};
    const int64_t obytes[3] = {gbytes, 4, pix * 12};
    const void* ins[3] = {derived, topk, target};
    const int64_t ibytes[3] = {gbytes, pix * K * (id_bits / 8), pix * 12};
    for (int o = 0; o < 3; ++o) {
        for (int q = 0; q < 3; ++q)
            if (overlap(outs[o], obytes[o], ins[q], ibytes[q])) return SAD_EINVAL;
        for (int q = o + 1; q < 3; ++q)
            if (overlap(outs[o], obytes[o], outs[q], obytes[q])) return SAD_EINVAL;
    }
    b.derived = derived;
    b.topk = topk;
    b.target = target;
    b.grad = grad;
    b.loss = loss;
    b.image = image;
    b.n = n;
    b.h = h;
    b.w = w;
    b.rg = region_grid(h, w);
    b.inv_p = pix > 0 ? 1.0 / ((double)h * (double)w) : 0.0;
    return SAD_OK;
}

inline int bwd_launch(const BwdArgs& b, void* stream) {
    const size_t nreg = (size_t)b.rg.rgx * b.rg.rgy;
    clear_error();
    hipLaunchKernelGGL(k_backward, dim3((unsigned)nreg), dim3(BWD_THREADS), 0, as_stream(stream), b);
    return launch_status();
}

}  // namespace sad

using namespace sad;

extern "C" int sad_render_bwd(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                              const float* target, float* grad, float* loss, float* image, void* stream) {
    BwdArgs b;
    const int st = bwd_setup(derived, n, h, w, topk, target, grad, loss, image, b);
    if (st != SAD_OK) return st;
    if (int64_t(h) * w == 0) return SAD_OK;
    return bwd_launch(b, stream);
}

// Checks and launch of the fused last pass + backward (the new lists are
// written with 32-bit ids, or 16-bit ones for the next step's first pass).
static int step_fused(const float* derived, int32_t n, int32_t h, int32_t w, const sad_pass_maps& m, int32_t stride,
                      uint64_t seed, uint32_t pass_index, int32_t inject_per_tile, const float* target, float* grad,
                      float* loss, float* image, void* stream) {
    // the pass writes lists and, optionally, all their logits: nothing else
    if (m.thr_next || m.probe_next) return SAD_EINVAL;
    PropArgs pa;
    int st = prop_setup(derived, n, h, w, m, stride, seed, pass_index, inject_per_tile, pa);
    if (st != SAD_OK) return st;
    const bool next16 = pa.next16 != nullptr;
    BwdArgs b;
    st = bwd_setup(derived, n, h, w, static_cast<const uint32_t*>(m.topk_next), target, grad, loss, image, b,
                   m.next_bits);
    if (st != SAD_OK) return st;
    // the pass's outputs must not share memory with anything else the step reads or writes
    const int64_t pix = int64_t(h) * w, gbytes = int64_t(n) * REC * 4;
    const void* outs[2] = {m.topk_next, m.scores_next};
    const int64_t mbytes[2] = {pix * K * (next16 ? 2 : 4), pix * K * 4};
    const void* others[5] = {target, grad, loss, image, derived};
    const int64_t obytes[5] = {pix * 12, gbytes, 4, pix * 12, gbytes};
    for (int o = 0; o < 2; ++o)
        for (int q = 0; q < 5; ++q)
            if (overlap(outs[o], mbytes[o], others[q], obytes[q])) return SAD_EINVAL;
    // nor may the backward's outputs share memory with the pass's inputs
    const void* bouts[3] = {grad, loss, image};
    const int64_t bbytes[3] = {gbytes, 4, pix * 12};
    const void* pins[4] = {m.topk_prev, m.scores_prev, m.thr_prev, m.probe_prev};
    const int64_t pbytes[4] = {pix * K * (m.prev_bits / 8), pix * K * 4, pix * 4, int64_t(n) * 16};
    for (int o = 0; o < 3; ++o)
        for (int q = 0; q < 4; ++q)
            if (overlap(bouts[o], bbytes[o], pins[q], pbytes[q])) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    // every check has passed: one kernel, one workgroup per backward region
    const size_t nreg = (size_t)b.rg.rgx * b.rg.rgy;
    const hipStream_t s = as_stream(stream);
    clear_error();
    const dim3 grid((unsigned)nreg), block(BWD_THREADS);
    const bool thr = pa.prev_thr != nullptr;
    if (pa.n > SMALL_IDS_MAX) {  // 32-bit maps only (prop_setup refuses 16-bit ones)
        if (thr)
            hipLaunchKernelGGL((k_step_last<false, false, true, false>), grid, block, 0, s, pa, b);
        else
            hipLaunchKernelGGL((k_step_last<false, false, false, false>), grid, block, 0, s, pa, b);
    } else if (next16) {  // the lists go to the next step's first pass
        if (pa.prev16 && thr)
            hipLaunchKernelGGL((k_step_last<true, true, true, true>), grid, block, 0, s, pa, b);
        else if (pa.prev16)
            hipLaunchKernelGGL((k_step_last<true, true, false, true>), grid, block, 0, s, pa, b);
        else if (thr)
            hipLaunchKernelGGL((k_step_last<true, false, true, true>), grid, block, 0, s, pa, b);
        else
            hipLaunchKernelGGL((k_step_last<true, false, false, true>), grid, block, 0, s, pa, b);
    } else if (pa.prev16) {
        if (thr)
            hipLaunchKernelGGL((k_step_last<true, true, true, false>), grid, block, 0, s, pa, b);
        else
            hipLaunchKernelGGL((k_step_last<true, true, false, false>), grid, block, 0, s, pa, b);
    } else {
        if (thr)
            hipLaunchKernelGGL((k_step_last<true, false, true, false>), grid, block, 0, s, pa, b);
        else
            hipLaunchKernelGGL((k_step_last<true, false, false, false>), grid, block, 0, s, pa, b);
    }
    return launch_status();
}

extern "C" int sad_step_fused(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk_prev,
                              const float* scores_prev, uint32_t* topk_next, float* scores_next, int32_t stride,
                              uint64_t seed, uint32_t pass_index, int32_t inject_per_tile, const float* target,
                              float* grad, float* loss, float* image, void* stream) {
    return step_fused(derived, n, h, w, maps32(topk_prev, scores_prev, topk_next, scores_next), stride, seed,
                      pass_index, inject_per_tile, target, grad, loss, image, stream);
}

extern "C" int sad_step_fused_pass(const float* derived, int32_t n, int32_t h, int32_t w, const sad_pass_maps* maps,
                                   int32_t stride, uint64_t seed, uint32_t pass_index, int32_t inject_per_tile,
                                   const float* target, float* grad, float* loss, float* image, void* stream) {
    if (!maps) return SAD_EINVAL;
    return step_fused(derived, n, h, w, *maps, stride, seed, pass_index, inject_per_tile, target, grad, loss, image,
                      stream);
}
