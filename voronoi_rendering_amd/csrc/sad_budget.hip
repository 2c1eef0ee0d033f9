// sad_budget.hip -- budget control: prune and split (Sec. 4.5, "Adaptive
// Budget: Densify and Prune"; Appendix B.5, "Densification scores", "Split
// kernel", "Pruning"), from the statistics of sad_site_stats.
//
// The rankings are stable radix sorts of per-site keys (the pages sort
// key-value pairs by radix): a float mapped to an unsigned integer of the
// same order, with the site id as the value, so equal keys keep ascending ids.
// Sites that do not take part get the largest key, so the ranked ones form a
// prefix of the sorted keys and no counts are needed; the free slots come
// from a stable select of the inactive ids.
//   1. prune: the n_prune active sites with the lowest removal delta are
//      switched off (position (-1, -1));
//   2. split: the sites still active with enough mass, ranked by
//      energy / mass^alpha (double), go in turn to the free slots in
//      ascending index; each parent becomes two children offset along the
//      major axis of its weighted covariance (or the target's Sobel gradient)
//      with the target colour, a smaller log tau and r, and zero Adam moments.
// The geometry is float32, one rounding per operation in the written order.
#include <algorithm>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_select.hpp>
#include <rocprim/iterator/counting_iterator.hpp>

#include "sad_device.h"
#include "sad_host.h"
#include "sad_prepare.h"

namespace sad {

constexpr int NSTAT_B = 8;

struct BudgetArgs {
    float* params;
    float* m;
    float* v;
    float* derived;
    const float* stats;
    const float* target;
    int32_t* done;  // nullable: [0] pruned, [1] split
    int32_t n, h, w, n_split, n_prune;
    float alpha, min_mass, offset, r_scale, logtau_shift;
    // workspace
    uint32_t *pkey, *pkey_s, *pid, *pid_s;          // prune ranking
    unsigned long long *skey, *skey_s;              // split ranking
    uint32_t *sid, *sid_s;
    uint8_t* free_flag;                             // [n] 1 for an inactive site
    uint32_t* slot;                                 // free slots, ascending
    int32_t* n_free;                                // [1] the number of free slots
    void* cub;                                      // the sorts' temporary storage
};

// unsigned integers with the order of the float (-0 as +0)
__device__ __forceinline__ uint32_t ordered32(float s) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ unsigned long long ordered64(double s) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(s + 0.0);
    return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ bool active_site(const float* params, int i) { return params[(size_t)i * REC] >= 0.0f; }

__global__ void k_budget_clear(int32_t* p, int k) {
    if ((int)threadIdx.x < k) p[threadIdx.x] = 0;
}

constexpr uint32_t NO_KEY32 = 0xFFFFFFFFu;  // larger than any active site's key (a NaN delta maps to +inf)
constexpr unsigned long long NO_KEY64 = ~0ull;

__global__ __launch_bounds__(256) void k_budget_prune_keys(BudgetArgs a) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0 && a.done) {
        a.done[0] = 0;
        a.done[1] = 0;
    }
    if (i >= a.n) return;
    const float dl = a.stats[(size_t)i * NSTAT_B + 2];
    a.pkey[i] = active_site(a.params, i) ? ordered32(dl == dl ? dl : __builtin_inff()) : NO_KEY32;
    a.pid[i] = (uint32_t)i;
}

// Thread k prunes the k-th ranked site; the ranked sites are a prefix of the
// sorted keys, so the last thread that prunes knows how many did.
__global__ __launch_bounds__(256) void k_budget_prune(BudgetArgs a) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    const int last = min(a.n_prune, a.n) - 1;
    if (k > last || a.pkey_s[k] == NO_KEY32) return;
    if (a.done && (k == last || a.pkey_s[k + 1] == NO_KEY32)) a.done[0] = k + 1;
    const uint32_t s = a.pid_s[k];
    float* p = a.params + (size_t)s * REC;
    p[0] = -1.0f;
    p[1] = -1.0f;
    const float4* q = reinterpret_cast<const float4*>(p);
    prepare_one(q[0], q[1], q[2], reinterpret_cast<float4*>(a.derived + (size_t)s * REC));
}

__global__ __launch_bounds__(256) void k_budget_split_keys(BudgetArgs a) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.n) return;
    const bool act = active_site(a.params, i);
    const float* st = a.stats + (size_t)i * NSTAT_B;
    const float mass = st[0];
    bool cand = act && (mass >= a.min_mass) && (mass > 0.0f);
    const double score = (double)st[1] / pow((double)mass, (double)a.alpha);
    cand = cand && (score == score);
    a.skey[i] = cand ? ~ordered64(score) : NO_KEY64;  // best first; ~ordered64 of a number is never ~0
    a.sid[i] = (uint32_t)i;
    a.free_flag[i] = act ? 0 : 1;
}

__device__ __forceinline__ float target_sum(const float* target, int h, int w, int i, int j) {
    i = i < 0 ? 0 : (i >= w ? w - 1 : i);
    j = j < 0 ? 0 : (j >= h ? h - 1 : j);
    const float* t = target + ((size_t)j * w + i) * 3;
    return (t[0] + t[1]) + t[2];
}

__device__ __forceinline__ int cell_of(float v, int size) {
    return (int)fminf(fmaxf(floorf(v), 0.0f), (float)(size - 1));
}

// Thread k splits the k-th ranked candidate into the k-th free slot.
__global__ __launch_bounds__(256) void k_budget_split(BudgetArgs a) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    const int last = min(a.n_split, *a.n_free) - 1;
    if (k > last || a.skey_s[k] == NO_KEY64) return;
    if (a.done && (k == last || a.skey_s[k + 1] == NO_KEY64)) a.done[1] = k + 1;
    const uint32_t pi = a.sid_s[k], ci = a.slot[k];
    float* pp = a.params + (size_t)pi * REC;
    float* pc = a.params + (size_t)ci * REC;
    const float* st = a.stats + (size_t)pi * NSTAT_B;
    const float* d = a.derived + (size_t)pi * REC;
    const int h = a.h, w = a.w;
    // the major axis of the weighted covariance about the site
    const float ms = st[0];
    const float mx = st[3] / ms, my = st[4] / ms;
    const float ca = st[5] / ms - mx * mx, cb = st[6] / ms - mx * my, cc = st[7] / ms - my * my;
    const float half = (ca - cc) * 0.5f;
    const float lam = (ca + cc) * 0.5f + __builtin_sqrtf(half * half + cb * cb);
    const float e1x = cb, e1y = lam - ca, e2x = lam - cc, e2y = cb;
    const float n1 = e1x * e1x + e1y * e1y, n2 = e2x * e2x + e2y * e2y;
    const bool first = n1 >= n2;
    const float ex = first ? e1x : e2x, ey = first ? e1y : e2y, nn = first ? n1 : n2;
    float ux, uy, sigma;
    if (lam > 0.0f && nn > 0.0f && finitef(lam) && finitef(nn)) {
        const float len = __builtin_sqrtf(nn);
        ux = ex / len;
        uy = ey / len;
        sigma = __builtin_sqrtf(lam);
    } else {
        // degenerate: the Sobel gradient of the target (channels summed) at the site's pixel
        const int i0 = cell_of(d[0], w), j0 = cell_of(d[1], h);
        const float gx = (target_sum(a.target, h, w, i0 + 1, j0 - 1) + 2.0f * target_sum(a.target, h, w, i0 + 1, j0) +
                          target_sum(a.target, h, w, i0 + 1, j0 + 1)) -
                         (target_sum(a.target, h, w, i0 - 1, j0 - 1) + 2.0f * target_sum(a.target, h, w, i0 - 1, j0) +
                          target_sum(a.target, h, w, i0 - 1, j0 + 1));
        const float gy = (target_sum(a.target, h, w, i0 - 1, j0 + 1) + 2.0f * target_sum(a.target, h, w, i0, j0 + 1) +
                          target_sum(a.target, h, w, i0 + 1, j0 + 1)) -
                         (target_sum(a.target, h, w, i0 - 1, j0 - 1) + 2.0f * target_sum(a.target, h, w, i0, j0 - 1) +
                          target_sum(a.target, h, w, i0 + 1, j0 - 1));
        const float gl = __builtin_sqrtf(gx * gx + gy * gy);
        ux = gl > 0.0f ? gx / gl : 1.0f;
        uy = gl > 0.0f ? gy / gl : 0.0f;
        sigma = 1.0f / fminf(d[6], d[7]);  // the larger scale
    }
    const float dx = (a.offset * sigma) * ux, dy = (a.offset * sigma) * uy;
    float base[REC];
#pragma unroll
    for (int q = 0; q < REC; ++q) base[q] = pp[q];
    const float x = base[0], y = base[1];
#pragma unroll
    for (int child = 0; child < 2; ++child) {
        float* o = child == 0 ? pp : pc;
        const uint32_t oi = child == 0 ? pi : ci;
        const float px = fminf(fmaxf(child == 0 ? x + dx : x - dx, 0.0f), (float)w);
        const float py = fminf(fmaxf(child == 0 ? y + dy : y - dy, 0.0f), (float)h);
        const float* t = a.target + ((size_t)cell_of(py, h) * w + cell_of(px, w)) * 3;
        float r[REC];
#pragma unroll
        for (int q = 0; q < REC; ++q) r[q] = base[q];
        r[0] = px;
        r[1] = py;
        r[2] = base[2] - a.logtau_shift;
        r[3] = base[3] * a.r_scale;
        r[4] = t[0];
        r[5] = t[1];
        r[6] = t[2];
        float4* o4 = reinterpret_cast<float4*>(o);
        o4[0] = make_float4(r[0], r[1], r[2], r[3]);
        o4[1] = make_float4(r[4], r[5], r[6], r[7]);
        o4[2] = make_float4(r[8], r[9], r[10], r[11]);
        float4* m4 = reinterpret_cast<float4*>(a.m + (size_t)oi * REC);
        float4* v4 = reinterpret_cast<float4*>(a.v + (size_t)oi * REC);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            m4[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            v4[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        prepare_one(make_float4(r[0], r[1], r[2], r[3]), make_float4(r[4], r[5], r[6], r[7]),
                    make_float4(r[8], r[9], r[10], r[11]), reinterpret_cast<float4*>(a.derived + (size_t)oi * REC));
    }
}

// rocPRIM's device radix sort: below its merge-sort limit (the default) it
// sorts blocks and merges them; a limit of 0 takes its onesweep path (one
// histogram, then one scatter kernel per 8-bit digit) at every size.
constexpr size_t SORT_MERGE_LIMIT = 1024 * 1024;
using SortConfig = rocprim::radix_sort_config<rocprim::default_config, rocprim::default_config,
                                              rocprim::default_config, SORT_MERGE_LIMIT>;

// Workspace layout for n sites; returns the total bytes (pointers filled when base != nullptr).
inline size_t budget_layout(int32_t n, char* base, BudgetArgs* a, size_t* cub_bytes) {
    size_t cb_p = 0, cb_s = 0, cb_f = 0;
    (void)rocprim::radix_sort_pairs<SortConfig>(nullptr, cb_p, (uint32_t*)nullptr, (uint32_t*)nullptr,
                                                (uint32_t*)nullptr, (uint32_t*)nullptr, (size_t)n, 0, 32);
    (void)rocprim::radix_sort_pairs<SortConfig>(nullptr, cb_s, (unsigned long long*)nullptr, (unsigned long long*)nullptr,
                                                (uint32_t*)nullptr, (uint32_t*)nullptr, (size_t)n, 0, 64);
    (void)rocprim::select(nullptr, cb_f, rocprim::counting_iterator<uint32_t>(0), (const uint8_t*)nullptr,
                          (uint32_t*)nullptr, (int32_t*)nullptr, (size_t)n);
    const size_t cub = std::max(cb_p, std::max(cb_s, cb_f));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += (bytes + 255) & ~(size_t)255;
        return p;
    };
    const size_t n4 = (size_t)n * 4, n8 = (size_t)n * 8;
    char* p[12];
    p[0] = take(n4); p[1] = take(n4); p[2] = take(n4); p[3] = take(n4);
    p[4] = take(n8); p[5] = take(n8); p[6] = take(n4); p[7] = take(n4);
    p[8] = take((size_t)n); p[9] = take(n4);
    p[10] = take(16);
    p[11] = take(cub);
    if (a) {
        a->pkey = (uint32_t*)p[0]; a->pkey_s = (uint32_t*)p[1]; a->pid = (uint32_t*)p[2]; a->pid_s = (uint32_t*)p[3];
        a->skey = (unsigned long long*)p[4]; a->skey_s = (unsigned long long*)p[5];
        a->sid = (uint32_t*)p[6]; a->sid_s = (uint32_t*)p[7];
        a->free_flag = (uint8_t*)p[8]; a->slot = (uint32_t*)p[9];
        a->n_free = (int32_t*)p[10];
        a->cub = p[11];
    }
    if (cub_bytes) *cub_bytes = cub;
    return off;
}

}  // namespace sad

using namespace sad;

extern "C" size_t sad_budget_workspace_bytes(int32_t n) {
    if (!sites_ok(n)) return 0;
    return budget_layout(n, nullptr, nullptr, nullptr);
}

extern "C" int sad_densify_prune(float* params, float* adam_m, float* adam_v, float* derived, int32_t n, int32_t h,
                                 int32_t w, const float* stats, const float* target, int32_t n_split, int32_t n_prune,
                                 float alpha, float min_mass, float offset, float r_scale, float logtau_shift,
                                 int32_t* done, void* workspace, size_t workspace_bytes, void* stream) {
    if (!sites_ok(n) || !image_ok(h, w) || n_split < 0 || n_prune < 0) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (n > 0 && pix == 0) return SAD_EINVAL;  // the split reads the target
    if (!array_ok(params, n, 16) || !array_ok(adam_m, n, 16) || !array_ok(adam_v, n, 16) ||
        !array_ok(derived, n, 16) || !array_ok(stats, n, 16) || !array_ok(target, n > 0 ? pix : 0, 4))
        return SAD_EINVAL;
    if (done && !aligned(done, 4)) return SAD_EINVAL;
    const size_t need = sad_budget_workspace_bytes(n);
    if (n > 0 && (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need)) return SAD_EINVAL;
    const int64_t rb = int64_t(n) * REC * 4, sb = int64_t(n) * NSTAT_B * 4;
    const void* bufs[8] = {params, adam_m, adam_v, derived, stats, target, done, workspace};
    const int64_t bytes[8] = {rb, rb, rb, rb, sb, n > 0 ? pix * 12 : 0, done ? 8 : 0, (int64_t)need};
    for (int x = 0; x < 8; ++x)
        for (int y = x + 1; y < 8; ++y)
            if (overlap(bufs[x], bytes[x], bufs[y], bytes[y])) return SAD_EINVAL;
    BudgetArgs a{};
    a.params = params;
    a.m = adam_m;
    a.v = adam_v;
    a.derived = derived;
    a.stats = stats;
    a.target = target;
    a.done = done;
    a.n = n;
    a.h = h;
    a.w = w;
    a.n_split = n_split;
    a.n_prune = n_prune;
    a.alpha = alpha;
    a.min_mass = min_mass;
    a.offset = offset;
    a.r_scale = r_scale;
    a.logtau_shift = logtau_shift;
    hipStream_t s = as_stream(stream);
    if (n == 0 && !done) return SAD_OK;
    clear_error();
    if (n == 0) {  // nothing to rank: both counts are 0
        hipLaunchKernelGGL(k_budget_clear, dim3(1), dim3(64), 0, s, done, 2);
        return launch_status();
    }
    size_t cub = 0;
    budget_layout(n, static_cast<char*>(workspace), &a, &cub);
    void* cub_tmp = a.cub;
    const unsigned g = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(k_budget_prune_keys, dim3(g), dim3(256), 0, s, a);
    size_t tb = cub;
    if (rocprim::radix_sort_pairs<SortConfig>(cub_tmp, tb, a.pkey, a.pkey_s, a.pid, a.pid_s, (size_t)n, 0, 32, s) !=
        hipSuccess)
        return SAD_EHIP;
    if (n_prune > 0)
        hipLaunchKernelGGL(k_budget_prune, dim3((unsigned)((std::min(n_prune, n) + 255) / 256)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_budget_split_keys, dim3(g), dim3(256), 0, s, a);
    tb = cub;
    if (rocprim::radix_sort_pairs<SortConfig>(cub_tmp, tb, a.skey, a.skey_s, a.sid, a.sid_s, (size_t)n, 0, 64, s) !=
        hipSuccess)
        return SAD_EHIP;
    tb = cub;
    if (rocprim::select(cub_tmp, tb, rocprim::counting_iterator<uint32_t>(0), a.free_flag, a.slot, a.n_free, (size_t)n,
                        s) != hipSuccess)
        return SAD_EHIP;
    if (n_split > 0)
        hipLaunchKernelGGL(k_budget_split, dim3((unsigned)((std::min(n_split, n) + 255) / 256)), dim3(256), 0, s, a);
    return launch_status();
}
