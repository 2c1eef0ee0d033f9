// sad_prepare.h -- the prepared record of one site (Sec. 4.1; format in
// sad.h): tau = exp(log tau), the rotation, the inverse scales, the colour;
// used by the preparation, Adam and budget kernels.
#pragma once

#include "sad_crmath.h"
#include "sad_device.h"

namespace sad {

constexpr float THETA_LIMIT = 1048576.0f;  // 2^20

// Prepared record of one site (format in sad.h); returns its geometry part.
__device__ __forceinline__ Geo prepare_one(const float4 p0, const float4 p1, const float4 p2, float4* out) {
    // p0 = (x, y, log_tau, r), p1 = (c_r, c_g, c_b, theta), p2 = (log_s1, log_s2, -, -)
    float theta = p1.w;
    bool active = p0.x >= 0.0f && fabsf(theta) <= THETA_LIMIT;
    float cs = 1.0f, sn = 0.0f;
    if (active) sincos_cr(theta, &sn, &cs);
    float4 o0, o1, o2;
    o0.x = active ? p0.x : -1.0f;
    o0.y = active ? p0.y : -1.0f;
    o0.z = exp_cr(p0.z);
    o0.w = p0.w;
    o1.x = cs;
    o1.y = sn;
    o1.z = exp_cr(-p2.x);
    o1.w = exp_cr(-p2.y);
    o2.x = p1.x;
    o2.y = p1.y;
    o2.z = p1.z;
    o2.w = 0.0f;
    out[0] = o0;
    out[1] = o1;
    out[2] = o2;
    Geo g;
    g.g0 = o0;
    g.g1 = o1;
    return g;
}

}  // namespace sad
