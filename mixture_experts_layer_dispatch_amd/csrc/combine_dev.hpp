// Gate-weighted combine work item (S10).
//
// MoE playbook (molayo1419.me, "How it works", combine step) and MoE lesson
// (factory.pai-world.com, "Mixture of Experts", "FFN swap"): the layer output is
// the gate-weighted sum of the chosen experts' outputs; the lesson's "Shared
// expert" section adds the always-on shared expert.  The sum is taken in fp32 in a
// fixed order -- routed experts in selection order, then the shared expert -- so
// results are bitwise reproducible, then rounded once to the output dtype.  A slot
// whose slot_to_row is negative (dropped by the capacity variant) is left out.
#pragma once

#include "common.hpp"

namespace moe {

// One lane: 16 bytes of output columns of one token; gid = t * (d / V) + column chunk.
template <bool F32, bool COH>
__device__ __forceinline__ void combine_lane(const void *__restrict__ yp, const int32_t *__restrict__ s2r,
                                             const float *__restrict__ gate, void *__restrict__ y, int T, int k,
                                             int d, int S, long gid) {
    constexpr int V = F32 ? 4 : 8;  // elements per 16-byte access
    const int per = d / V;
    const long t = gid / per;
    if (t >= T) return;
    const int c = (int)(gid % per) * V;
    const long tk = (long)T * k;
    float acc[V];
#pragma unroll
    for (int u = 0; u < V; ++u) acc[u] = 0.0f;
    auto add_row = [&](const i32x4 &q, float g, bool scale) {
        if constexpr (F32) {
            float v[4] = {__int_as_float(q[0]), __int_as_float(q[1]), __int_as_float(q[2]), __int_as_float(q[3])};
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] = scale ? acc[u] + g * v[u] : acc[u] + v[u];
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float v = bf16_to_f32((uint16_t)((uint32_t)q[u >> 1] >> (16 * (u & 1))));
                acc[u] = scale ? acc[u] + g * v : acc[u] + v;
            }
        }
    };
    // All loads of a chunk of choices are issued before any is used (clamped, unconditional:
    // a load under a branch would be waited for before the branch joins), the shared row's
    // with the first chunk; the additions keep the fixed order.
    constexpr int CH = 8;
    const size_t esz = F32 ? 4 : 2;
    const i32x4 qs = S ? ldc16<COH>(yp, (size_t)((tk + t) * d + c) * esz) : (i32x4){0, 0, 0, 0};
    for (int j0 = 0; j0 < k; j0 += CH) {
        long r[CH];
        float g[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int j = j0 + u < k ? j0 + u : k - 1;
            r[u] = ldc<COH>(s2r + t * k + j);
            g[u] = ldc<COH>(gate + t * k + j);
        }
        i32x4 q[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const long rr = r[u] < 0 ? 0 : (r[u] >= tk ? tk - 1 : r[u]);
            q[u] = ldc16<COH>(yp, (size_t)(rr * d + c) * esz);
        }
        // a slot without a row (slot_to_row < 0: dropped by the capacity variant) adds nothing
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (j0 + u < k && r[u] >= 0) add_row(q[u], g[u], true);
    }
    if (S) add_row(qs, 1.0f, false);
    if constexpr (F32) {
        *(float4 *)((float *)y + t * d + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        *(uint4 *)((uint16_t *)y + t * d + c) = o;
    }
}

}  // namespace moe
