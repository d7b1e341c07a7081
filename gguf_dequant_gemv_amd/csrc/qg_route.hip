// qg_route.hip -- router top-k / expert grouping and the MoE combine (gfx950).
#include "qg_kernels.h"

namespace qg {

// -------------------------------------------------------------- router ----
// One wave per token: the k largest logits (ties to the lower index) in pick
// order, and exp(l_j - l_0) / sum over the picks.  The qwen3_moe_ssd.js topk
// kernel's selection and renormalisation; ranking logits orders as ranking
// the probabilities does.  With `grp` set it also groups the (token, pick)
// pairs by expert for the expert GEMVs (slot lookup, absent-expert status).
// NS register sets of 64 experts per lane (E <= 64 NS).  Every global input
// goes out in one batch (the wave's logits, then the experts' slots and down
// scales into LDS), so the launch pays one memory round trip before the
// selection.
template <int NS>
__global__ __launch_bounds__(1024) void k_route(const float *logits, int E, int k, int T,
                                                const int32_t *slots, int n_slots, int32_t *ids_out, float *w_out,
                                                int32_t *status, int32_t *rt_ids, float *rt_w,
                                                int32_t *rt_valid, int32_t *grp, int ca, int32_t *sets_a, int cb,
                                                int32_t *sets_b, const float *escale, int32_t *rt_pslot,
                                                float *rt_pes) {
    __shared__ int s_ids[MAXT * 32];
    __shared__ int s_valid[MAXT];
    __shared__ u32 s_tmask[256];    // expert e: bit t set when valid token t picked e
    __shared__ int s_gidx[256];     // expert e: its group index
    __shared__ int s_wcnt[16];
    __shared__ int s_slot[256];     // expert e: its pool slot
    __shared__ float s_es[256];     // expert e: its down scale (1 without one)
    __shared__ float s_val[MAXT * 32];
    __shared__ int s_na[256], s_nb[256];   // set lists: chunks per group, then their running sums
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    float lv[NS] = {};
    if (wave < T) {
        const float *l = logits + (int64_t)wave * E;
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const int e = lane + 64 * i;
            lv[i] = e < E ? l[e] : 0.0f;
        }
    }
    const bool want_es = rt_pslot && escale;
    for (int e = tid; e < E; e += blockDim.x) {
        const int sv = slots ? slots[e] : 0;
        const float ev = want_es ? escale[e] : 1.0f;
        s_tmask[e] = 0u;
        s_slot[e] = sv;
        s_es[e] = ev;
    }
    if (wave < T) {
        u32 key[NS];
        u32 taken = 0u;  // bit i: value lane + 64 i is picked or absent
#pragma unroll
        for (int i = 0; i < NS; i++) {
            key[i] = order_key(lv[i]);
            if (lane + 64 * i >= E) taken |= 1u << i;
        }
        for (int j = 0; j < k; j++) {
            // the largest key still free; among equal keys the lowest index
            u32 lm = 0u;
#pragma unroll
            for (int i = 0; i < NS; i++)
                if (!((taken >> i) & 1u)) lm = max(lm, key[i]);
            const u32 M = wave_max_u32(lm);
            int e = -1;
#pragma unroll
            for (int i = 0; i < NS; i++) {
                const unsigned long long b = __ballot(!((taken >> i) & 1u) && key[i] == M);
                if (e < 0 && b) e = 64 * i + (int)__builtin_ctzll(b);
            }
            if ((e & 63) == lane) {
                taken |= 1u << (e >> 6);
                float v = lv[0];
#pragma unroll
                for (int i = 1; i < NS; i++) v = (e >> 6) == i ? lv[i] : v;
                s_ids[wave * k + j] = e;
                s_val[wave * k + j] = v;
            }
        }
    }
    __syncthreads();   // picks, logit values and slots visible to every wave
    if (wave < T) {
        // weights over the picks, relative to the top pick
        float ex = 0.0f;
        const float l0 = s_val[wave * k];
        int ok = 1;
        if (lane < k) {
            const int id = s_ids[wave * k + lane];
            ex = expf(s_val[wave * k + lane] - l0);
            const int sl = s_slot[id];
            ok = sl >= 0 && sl < n_slots;
            if (rt_pslot) {   // each pick's slot and down scale, pick order
                rt_pslot[wave * k + lane] = sl;
                rt_pes[wave * k + lane] = s_es[id];
            }
        }
        const float sum = wave_sum(ex);
        const int all_ok = __ballot(!ok) == 0ull;
        if (lane < k) {
            const float wj = ex / sum;
            const int z = wave * k + lane;
            if (rt_ids) rt_ids[z] = s_ids[z];
            if (rt_w) rt_w[z] = wj;
            if (ids_out) ids_out[z] = s_ids[z];
            if (w_out) w_out[z] = wj;
        }
        if (lane == 0) {
            s_valid[wave] = all_ok;
            if (rt_valid) rt_valid[wave] = all_ok;
        }
    }
    __syncthreads();
    if (!grp) return;
    // Group pairs by expert: ascending expert id, pairs in (t, j) order.  A
    // token picks an expert at most once, so a pair's place in its group is
    // the number of lower tokens that picked the same expert.
    for (int z = tid; z < T * k; z += blockDim.x) {
        const int t = z / k;
        if (s_valid[t]) atomicOr(&s_tmask[s_ids[z]], 1u << t);
    }
    __syncthreads();
    const bool has = tid < E && s_tmask[tid] != 0u;
    const unsigned long long mask = __ballot(has);
    if (lane == 0) s_wcnt[wave] = __popcll(mask);
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wave; w2++) base += s_wcnt[w2];
    const int gi = base + __popcll(mask & ((1ull << lane) - 1ull));
    if (tid == 0) {
        int ok = 1, G = 0;
        for (int t = 0; t < T; t++) ok &= s_valid[t];
        for (int w2 = 0; w2 < (int)(blockDim.x >> 6); w2++) G += s_wcnt[w2];
        if (status) *status = ok ? 0 : -2;  // QG_OK / QG_EABSENT
        grp[0] = G;
    }
    if (has) {
        int *rec = grp + 1 + gi * GREC;
        rec[0] = tid;
        rec[1] = s_slot[tid];
        rec[2] = __popc(s_tmask[tid]);
        s_gidx[tid] = gi;
    }
    __syncthreads();
    for (int z = tid; z < T * k; z += blockDim.x) {
        const int t = z / k;
        if (!s_valid[t]) continue;
        const int e = s_ids[z];
        const int r = __popc(s_tmask[e] & ((1u << t) - 1u));
        int *rec = grp + 1 + s_gidx[e] * GREC;
        rec[3 + r] = t;
        rec[19 + r] = z;
    }
    if (!sets_a && !sets_b) return;
    // Set lists: group g holds ceil(n_g / c) chunks of c pairs; the chunks go
    // out in group order at the running sum of the lower groups' counts
    // (inclusive scan over the experts, whose order is the groups' order).
    const int n = has ? __popc(s_tmask[tid]) : 0;
    if (tid < 256) {
        s_na[tid] = sets_a ? (n + ca - 1) / ca : 0;
        s_nb[tid] = sets_b ? (n + cb - 1) / cb : 0;
    }
    __syncthreads();
    if (wave == 0) {   // inclusive scans of both, by one wave: 4 experts a lane, then across the lanes
        int a4[4], b4[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a4[i] = s_na[4 * lane + i];
            b4[i] = s_nb[4 * lane + i];
        }
#pragma unroll
        for (int i = 1; i < 4; i++) {
            a4[i] += a4[i - 1];
            b4[i] += b4[i - 1];
        }
        int ta = a4[3], tb = b4[3];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int ua = __shfl_up(ta, d), ub = __shfl_up(tb, d);
            if (lane >= d) {
                ta += ua;
                tb += ub;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            s_na[4 * lane + i] = ta - a4[3] + a4[i];
            s_nb[4 * lane + i] = tb - b4[3] + b4[i];
        }
    }
    __syncthreads();
    if (has) {
        if (sets_a) {
            const int c1 = s_na[tid], c0 = tid ? s_na[tid - 1] : 0;
            for (int c = c0; c < c1; c++) sets_a[1 + c] = (gi << 16) | ((c - c0) * ca);
        }
        if (sets_b) {
            const int c1 = s_nb[tid], c0 = tid ? s_nb[tid - 1] : 0;
            for (int c = c0; c < c1; c++) sets_b[1 + c] = (gi << 16) | ((c - c0) * cb);
        }
    }
    if (tid == 0) {
        if (sets_a) sets_a[0] = s_na[255];
        if (sets_b) sets_b[0] = s_nb[255];
    }
}

// ------------------------------------------------------------- combine ----
// y[t][h] = sum_j dn'[t*k + j][h], added in pick order, where the down launch
// already stored dn' = (dn * s[id]) * w_j (the gemma4_moe_ssd.js moeSum /
// qwen3_moe_ssd.js moeAccum combine, same operations in the same order);
// tokens with an absent pick are left untouched.
__global__ __launch_bounds__(256) void k_combine(const float *dn, const int32_t *rt_valid, float *y, int64_t H,
                                                 int k) {
    const int t = blockIdx.y;
    const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    const int ok = rt_valid[t];
    const float *p = dn + (int64_t)t * k * H + h;
    float acc = 0.0f;
    // eight picks' loads in flight at a time, added in pick order
    for (int j0 = 0; j0 < k; j0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = j0 + j < k ? p[(int64_t)(j0 + j) * H] : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++)
            if (j0 + j < k) acc += v[j];
    }
    if (ok) y[(int64_t)t * H + h] = acc;
}

route_fn route_kernel(int E) { return E <= 64 ? k_route<1> : E <= 128 ? k_route<2> : k_route<4>; }

}  // namespace qg
