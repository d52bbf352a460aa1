// specverify.hip -- gfx950 kernels and C ABI of the verify-and-accept step
// (Leviathan rejection sampling over chains and flattened draft trees).
//
// Pages followed (title and section):
//   [PT] "Decodificacao Especulativa e EAGLE-3" (ai-engineering.academy):
//        "O Conceito" (accept with min(1, q/p), first rejection -> residual,
//        all accepted -> bonus from q_{N+1}); Implementando, Passo 1 (accept
//        rule) and Passo 2 (residual (q-p)_+ normalised, q if it is zero).
//   [ZH] "投机解码与 EAGLE：步骤、发展历史与三代差异" (caijizhuo.github.io):
//        section 3 (flattened tree, one verifier pass) and section 4
//        ("eagle_round" step 4, the walk from the root).
//
// One call is four kernels on the caller's stream:
//   1. row statistics: every q/p row the accept tests read is streamed once
//      (16-byte loads, 4 in flight per thread); per row (m, s) with
//      s = sum exp((z - m)/T) from the hardware exp2 in fp32, summed in
//      pairs of 32 and accumulated in double.  This is the HBM-bound pass.
//   2. accept: one wave64 per chain (lane i = position i+1; ballot + ffs
//      finds the first rejection) or one block per tree (every node tested
//      in parallel, then a wave walks the parent array with ballots).  The
//      ratio q(d)/p(d) is formed in double from the row statistics.
//   3. sampling partials: the one or two rows the sample needs are split in
//      4096-element chunks; each block evaluates its chunk in double (exp of
//      (z - m)/T per element) and writes chunk sums.
//   4. sampling final: one block per sequence combines the chunk sums, finds
//      the chunk holding u*W, rescans it with a block-wide prefix scan and
//      writes the token (inverse CDF in token order).
// The residual avoids a third sweep: with pass-1 statistics it decides which
// tokens have q > p (a log-domain comparison), accumulates sum a_t, sum b_t
// and the same two sums over that set in double, and forms
// W = sum_{q>p} a_t - (Sq/Sp) sum_{q>p} b_t once the exact Sq, Sp are known.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.h"
#include "specverify.h"

namespace sv {

// ===========================================================================
// 1. Row statistics
// ===========================================================================
template <int K>
__device__ __forceinline__ void accumulate_values(const float* x, float c, double cd, float& ref, double& acc)
{
    float lm = x[0];
#pragma unroll
    for (int i = 1; i < K; ++i) lm = fmaxf(lm, x[i]);
    // move the reference when the first finite value arrives or the maximum
    // grows by more than one binary order of magnitude: the terms that
    // dominate the sum then have exponent arguments in (-few, 1], where the
    // fp32 rounding of (x - ref) * c is smallest
    if ((lm - ref) * c > 1.0f) {
        acc = (ref == -INFINITY) ? 0.0 : acc * exp2((double)(ref - lm) * cd);
        ref = lm;
    }
    const float r = (ref == -INFINITY) ? 0.0f : ref;
    float e[K];
#pragma unroll
    for (int i = 0; i < K; ++i) e[i] = __builtin_amdgcn_exp2f((x[i] - r) * c);
#pragma unroll
    for (int w = 1; w < K; w <<= 1) {
#pragma unroll
        for (int i = 0; i + w < K; i += 2 * w) e[i] += e[i + w];
    }
    acc += (double)e[0];
}

__device__ __forceinline__ void combine_stat(float& m, double& s, float m2, double s2, double cd)
{
    const float M = fmaxf(m, m2);
    const double f1 = (m == M) ? 1.0 : exp2((double)(m - M) * cd);
    const double f2 = (m2 == M) ? 1.0 : exp2((double)(m2 - M) * cd);
    s = s * f1 + s2 * f2;
    m = M;
}

// (m, s) of one row, valid in thread 0.
template <int DT, int U>
__device__ __forceinline__ RowStat block_row_stats(const char* __restrict__ row, int V, float c, double cd)
{
    constexpr int EB = elem_bytes<DT>();
    constexpr int EPV = 16 / EB;
    float ref = -INFINITY;
    double acc = 0.0;
    // elements before the first 16-byte boundary (rows need only be
    // element-aligned); the rest of the row streams as 16-byte vectors
    int head = (int)(((16u - ((uint32_t)(uintptr_t)row & 15u)) & 15u) / EB);
    head = head < V ? head : V;
    if ((int)threadIdx.x < head) {
        float x[1] = {load_logit<DT>(row, threadIdx.x)};
        accumulate_values<1>(x, c, cd, ref, acc);
    }
    row += head * EB;
    V -= head;
    const int nvec = V / EPV;
    const uint4* __restrict__ vrow = reinterpret_cast<const uint4*>(row);
    int v = threadIdx.x;
    for (; v + (U - 1) * kBlock < nvec; v += U * kBlock) {
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = vrow[v + u * kBlock];
        float x[U * EPV];
#pragma unroll
        for (int u = 0; u < U; ++u) decode16<DT>(raw[u], x + u * EPV);
        accumulate_values<U * EPV>(x, c, cd, ref, acc);
    }
    for (; v < nvec; v += kBlock) {
        float x[EPV];
        decode16<DT>(vrow[v], x);
        accumulate_values<EPV>(x, c, cd, ref, acc);
    }
    const int tail = V - nvec * EPV;
    if ((int)threadIdx.x < tail) {
        float x[1] = {load_logit<DT>(row, (int64_t)nvec * EPV + threadIdx.x)};
        accumulate_values<1>(x, c, cd, ref, acc);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(ref, off, 64);
        const double s2 = __shfl_xor(acc, off, 64);
        combine_stat(ref, acc, m2, s2, cd);
    }
    __shared__ float red_m[kWaves];
    __shared__ double red_s[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red_m[wave] = ref;
        red_s[wave] = acc;
    }
    __syncthreads();
    RowStat st;
    st.m = red_m[0];
    st.s = red_s[0];
    st.pad = 0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kWaves; ++w) combine_stat(st.m, st.s, red_m[w], red_s[w], cd);
    }
    return st;
}

// Chain: block r covers row j = r % (2N) of sequence b = r / (2N): q row j
// for j < N, else p row j - N.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_stats_chain(const char* __restrict__ zq, int64_t qs, int64_t qr,
                                                        const char* __restrict__ zp, int64_t ps, int64_t pr, int N,
                                                        int V, float c, double cd, RowStat* __restrict__ stats)
{
    constexpr int EB = elem_bytes<DT>();
    const int row = blockIdx.x;
    const int b = row / (2 * N);
    const int j = row - b * 2 * N;
    const char* base = (j < N) ? zq + ((int64_t)b * qs + (int64_t)j * qr) * EB
                               : zp + ((int64_t)b * ps + (int64_t)(j - N) * pr) * EB;
    const RowStat st = block_row_stats<DT, 4>(base, V, c, cd);
    if (threadIdx.x == 0) stats[row] = st;
}

// Tree: block r covers node n of sequence b, q (which 0) or p (which 1);
// nodes without children are skipped (their rows are never tested against).
template <int DT>
__global__ __launch_bounds__(kBlock) void k_stats_tree(const char* __restrict__ zq, int64_t qs, int64_t qr,
                                                       const char* __restrict__ zp, int64_t ps, int64_t pr,
                                                       const int32_t* __restrict__ parents, int parents_shared,
                                                       int nn, int V, float c, double cd,
                                                       RowStat* __restrict__ stats)
{
    constexpr int EB = elem_bytes<DT>();
    const int row = blockIdx.x;  // (b * nn + n) * 2 + which
    const int which = row & 1;
    const int bn = row >> 1;
    const int b = bn / nn;
    const int n = bn - b * nn;
    const int32_t* par = parents_shared ? parents : parents + (int64_t)b * nn;
    int found = 0;
    for (int m = n + 1 + (int)threadIdx.x; m < nn; m += kBlock) found |= (par[m] == n);
    if (!__syncthreads_or(found)) return;
    const char* base = which == 0 ? zq + ((int64_t)b * qs + (int64_t)n * qr) * EB
                                  : zp + ((int64_t)b * ps + (int64_t)n * pr) * EB;
    const RowStat st = block_row_stats<DT, 4>(base, V, c, cd);
    if (threadIdx.x == 0) stats[row] = st;
}

__device__ __forceinline__ bool stat_bad(const RowStat& r) { return !(r.s > 0.0 && r.s < INFINITY); }

// ===========================================================================
// 2. Accept
// ===========================================================================
struct AcceptOut {
    double lq, lp;  // log q(d), log p(d)
    int accepted;
};

template <int DT>
__device__ __forceinline__ AcceptOut accept_one(const char* qrow, const char* prow, int tok, const RowStat& rq,
                                                const RowStat& rp, double invT, double u)
{
    const float zqd = load_logit<DT>(qrow, tok);
    const float zpd = load_logit<DT>(prow, tok);
    AcceptOut o;
    o.lq = ((double)zqd - (double)rq.m) * invT - log(rq.s);
    o.lp = ((double)zpd - (double)rp.m) * invT - log(rp.s);
    if (zpd == -INFINITY) {
        o.accepted = 1;  // zero draft probability
    } else {
        const double r = exp(o.lq - o.lp);
        o.accepted = u < fmin(1.0, r) ? 1 : 0;
    }
    return o;
}

__device__ __forceinline__ void fill_residual_state(SeqState& s, const RowStat& rq, const RowStat& rp, float T)
{
    s.mode = kModeResidual;
    s.mq = rq.m;
    s.mp = rp.m;
    s.sq = rq.s;
    s.sp = rp.s;
    const double theta = ((double)rq.m - (double)rp.m) + (double)T * (log(rq.s) - log(rp.s));
    // margin: pass-1 sums carry a relative error well below 1e-6 each; the
    // margin covers ten times that plus the fp32 rounding of theta
    const double margin = 4e-6 * (double)T + 2.5e-7 * fabs(theta) + 1e-30;
    s.thr_lo = (float)(theta - margin);
    s.thr_hi = (float)(theta + margin);
}

// One wave64 per chain; lane i handles position i+1.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_accept_chain(
    const char* __restrict__ zq, int64_t qs, int64_t qr, const char* __restrict__ zp, int64_t ps, int64_t pr,
    const int32_t* __restrict__ d, int B, int N, int V, uint64_t seed, uint64_t round, double invT, float T,
    const RowStat* __restrict__ stats, SeqState* __restrict__ st, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_num, int8_t* __restrict__ out_acc, float* __restrict__ out_probs)
{
    constexpr int EB = elem_bytes<DT>();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int b = blockIdx.x * kWaves + wave;
    if (b >= B) return;  // whole wave
    const int width = N + 1;
    const bool active = lane < N;
    int err = 0, acc = 1;
    RowStat rq{}, rp{};
    if (active) {
        const int tok = d[(int64_t)b * N + lane];
        rq = stats[(int64_t)b * 2 * N + lane];
        rp = stats[(int64_t)b * 2 * N + N + lane];
        if (tok < 0 || tok >= V || stat_bad(rq) || stat_bad(rp)) {
            err = 1;
        } else {
            const double u = accept_uniform(seed, round, (uint32_t)b, (uint32_t)(lane + 1));
            const AcceptOut o = accept_one<DT>(zq + ((int64_t)b * qs + (int64_t)lane * qr) * EB,
                                               zp + ((int64_t)b * ps + (int64_t)lane * pr) * EB, tok, rq, rp,
                                               invT, u);
            acc = o.accepted;
            if (out_probs) {
                out_probs[((int64_t)b * N + lane) * 2 + 0] = (float)exp(o.lq);
                out_probs[((int64_t)b * N + lane) * 2 + 1] = (float)exp(o.lp);
            }
        }
    }
    const uint64_t errmask = __ballot(err);
    const uint64_t rejmask = __ballot(active && !acc);
    if (errmask) {
        for (int i = lane; i < width; i += 64) out_tokens[(int64_t)b * width + i] = -1;
        if (lane == 0) {
            out_num[b] = -1;
            st[b].status = 1;
        }
        return;
    }
    const int k = rejmask ? (__ffsll((unsigned long long)rejmask) - 1) : N;
    if (active && out_acc) out_acc[(int64_t)b * N + lane] = (int8_t)acc;
    for (int i = lane; i < width; i += 64) out_tokens[(int64_t)b * width + i] = (i < k) ? d[(int64_t)b * N + i] : -1;
    // statistics of row k (residual) travel from lane k
    RowStat kq, kp;
    kq.m = __shfl(rq.m, k < N ? k : 0, 64);
    kq.s = __shfl(rq.s, k < N ? k : 0, 64);
    kp.m = __shfl(rp.m, k < N ? k : 0, 64);
    kp.s = __shfl(rp.s, k < N ? k : 0, 64);
    if (lane == 0) {
        out_num[b] = k;
        SeqState s{};
        s.k = k;
        s.status = 0;
        s.u = sample_uniform(seed, round, (uint32_t)b, (uint32_t)(k + 1));
        s.q_off = (int64_t)b * qs + (int64_t)k * qr;
        if (k < N) {
            s.p_off = (int64_t)b * ps + (int64_t)k * pr;
            fill_residual_state(s, kq, kp, T);
        } else {
            s.p_off = 0;
            s.mode = kModeBonus;
        }
        st[b] = s;
    }
}

// One block per tree: every node n >= 1 is tested against its parent's q/p
// rows, then wave 0 walks from the root into the lowest-index accepted child.
constexpr int kMaxNodes = 1024;

template <int DT>
__global__ __launch_bounds__(kBlock) void k_accept_tree(
    const char* __restrict__ zq, int64_t qs, int64_t qr, const char* __restrict__ zp, int64_t ps, int64_t pr,
    const int32_t* __restrict__ node_tokens, const int32_t* __restrict__ parents, int parents_shared, int B, int T,
    int V, int max_depth, uint64_t seed, uint64_t round, double invT, float temp, const RowStat* __restrict__ stats,
    SeqState* __restrict__ st, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_path,
    int32_t* __restrict__ out_num, int8_t* __restrict__ out_acc, float* __restrict__ out_probs)
{
    constexpr int EB = elem_bytes<DT>();
    const int b = blockIdx.x;
    const int nn = T + 1;
    const int width = max_depth + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int s_par[kMaxNodes];
    __shared__ unsigned char s_acc[kMaxNodes];
    __shared__ unsigned char s_kids[kMaxNodes];
    const int32_t* par = parents_shared ? parents : parents + (int64_t)b * nn;
    const int32_t* tok = node_tokens + (int64_t)b * nn;
    for (int n = tid; n < nn; n += kBlock) {
        s_kids[n] = 0;
        s_acc[n] = 0;
    }
    __syncthreads();
    int err = 0;
    for (int n = tid; n < nn; n += kBlock) {
        const int p = (n == 0) ? -1 : par[n];
        s_par[n] = p;
        if (n >= 1) {
            if (p < 0 || p >= n) err = 1;
            else s_kids[p] = 1;
            const int t = tok[n];
            if (t < 0 || t >= V) err = 1;
        }
    }
    err = __syncthreads_or(err);
    if (!err) {
        for (int n = 1 + tid; n < nn; n += kBlock) {
            const int p = s_par[n];
            const RowStat rq = stats[((int64_t)b * nn + p) * 2 + 0];
            const RowStat rp = stats[((int64_t)b * nn + p) * 2 + 1];
            if (stat_bad(rq) || stat_bad(rp)) {
                err = 1;
                continue;
            }
            const double u = accept_uniform(seed, round, (uint32_t)b, (uint32_t)n);
            const AcceptOut o = accept_one<DT>(zq + ((int64_t)b * qs + (int64_t)p * qr) * EB,
                                               zp + ((int64_t)b * ps + (int64_t)p * pr) * EB, tok[n], rq, rp, invT,
                                               u);
            s_acc[n] = (unsigned char)o.accepted;
            if (out_acc) out_acc[(int64_t)b * nn + n] = (int8_t)o.accepted;
            if (out_probs) {
                out_probs[((int64_t)b * nn + n) * 2 + 0] = (float)exp(o.lq);
                out_probs[((int64_t)b * nn + n) * 2 + 1] = (float)exp(o.lp);
            }
        }
    }
    err = __syncthreads_or(err);
    if (err) {
        for (int i = tid; i < width; i += kBlock) {
            out_tokens[(int64_t)b * width + i] = -1;
            out_path[(int64_t)b * width + i] = -1;
        }
        if (tid == 0) {
            out_num[b] = -1;
            st[b].status = 1;
        }
        return;
    }
    if (tid == 0) {
        if (out_acc) out_acc[(int64_t)b * nn] = 1;
        if (out_probs) {
            out_probs[(int64_t)b * nn * 2 + 0] = 0.0f;
            out_probs[(int64_t)b * nn * 2 + 1] = 0.0f;
        }
    }
    if (wave != 0) return;
    int cur = 0, depth = 0, residual = 0, werr = 0;
    for (;;) {
        if (!s_kids[cur]) break;  // leaf: bonus from q at cur
        int next = -1;
        for (int base = cur + 1; base < nn; base += 64) {
            const int n = base + lane;
            const bool pred = n < nn && s_par[n] == cur && s_acc[n];
            const uint64_t m = __ballot(pred);
            if (m) {
                next = base + __ffsll((unsigned long long)m) - 1;
                break;
            }
        }
        if (next < 0) {
            residual = 1;
            break;
        }
        if (depth + 1 > max_depth) {
            werr = 1;
            break;
        }
        ++depth;
        if (lane == 0) {
            out_path[(int64_t)b * width + depth] = next;
            out_tokens[(int64_t)b * width + depth - 1] = tok[next];
        }
        cur = next;
    }
    if (werr) {
        for (int i = lane; i < width; i += 64) {
            out_tokens[(int64_t)b * width + i] = -1;
            out_path[(int64_t)b * width + i] = -1;
        }
        if (lane == 0) {
            out_num[b] = -1;
            st[b].status = 1;
        }
        return;
    }
    for (int i = lane; i < width; i += 64) {
        if (i > depth) {
            out_tokens[(int64_t)b * width + i] = -1;
            out_path[(int64_t)b * width + i] = -1;
        }
    }
    if (lane == 0) {
        out_path[(int64_t)b * width] = 0;
        out_num[b] = depth;
        SeqState s{};
        s.k = depth;
        s.status = 0;
        s.u = sample_uniform(seed, round, (uint32_t)b, (uint32_t)(depth + 1));
        s.q_off = (int64_t)b * qs + (int64_t)cur * qr;
        if (residual) {
            s.p_off = (int64_t)b * ps + (int64_t)cur * pr;
            fill_residual_state(s, stats[((int64_t)b * nn + cur) * 2 + 0], stats[((int64_t)b * nn + cur) * 2 + 1],
                                temp);
        } else {
            s.p_off = 0;
            s.mode = kModeBonus;
        }
        st[b] = s;
    }
}

// ===========================================================================
// 3./4. Sampling
// ===========================================================================
// The 16 elements of thread `tid` in chunk `c` (contiguous, token order);
// entries past V read as -inf.
template <int DT>
__device__ __forceinline__ void load_chunk16(const char* __restrict__ row, int V, int c, int tid, float* x)
{
    const int64_t e0 = (int64_t)c * kChunk + (int64_t)tid * kPerThread;
    if (e0 + kPerThread <= V && (((uintptr_t)(row + e0 * elem_bytes<DT>())) & 15u) == 0) {
        const uint4* p = reinterpret_cast<const uint4*>(row + e0 * elem_bytes<DT>());
        constexpr int NV = kPerThread * elem_bytes<DT>() / 16;
        uint4 raw[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) raw[i] = p[i];
#pragma unroll
        for (int i = 0; i < NV; ++i) decode16<DT>(raw[i], x + i * (16 / elem_bytes<DT>()));
    } else {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) x[j] = (e0 + j < V) ? load_logit<DT>(row, e0 + j) : -INFINITY;
    }
}

// Chunk sums of the row(s) a sequence samples from (see ChunkSums).
template <int DT>
__global__ __launch_bounds__(kBlock) void k_sample_partials(const char* __restrict__ zq, const char* __restrict__ zp,
                                                            int V, int nchunks, double invT,
                                                            const SeqState* __restrict__ st,
                                                            ChunkSums* __restrict__ partials)
{
    constexpr int EB = elem_bytes<DT>();
    const int c = blockIdx.x, b = blockIdx.y;
    const SeqState s = st[b];
    if (s.status) return;
    __shared__ double red[kWaves];
    __shared__ float redf[kWaves];
    float xq[kPerThread];
    load_chunk16<DT>(zq + s.q_off * EB, V, c, threadIdx.x, xq);
    ChunkSums out;
    out.pad = 0.0;
    if (s.mode == kModeResidual) {
        float xp[kPerThread];
        load_chunk16<DT>(zp + s.p_off * EB, V, c, threadIdx.x, xp);
        double sa = 0.0, sb = 0.0, pa = 0.0, pb = 0.0, na = 0.0, nb = 0.0;
        float dmin = INFINITY, dmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const double a = exp(((double)xq[j] - (double)s.mq) * invT);
            const double bb = exp(((double)xp[j] - (double)s.mp) * invT);
            sa += a;
            sb += bb;
            const float d = xq[j] - xp[j];
            if (d > s.thr_hi) {
                pa += a;
                pb += bb;
            } else if (d >= s.thr_lo) {
                na += a;
                nb += bb;
                dmin = fminf(dmin, d);
                dmax = fmaxf(dmax, d);
            }
        }
        out.sa = block_sum(sa, red);
        out.sb = block_sum(sb, red);
        out.pa = block_sum(pa, red);
        out.pb = block_sum(pb, red);
        out.na = block_sum(na, red);
        out.nb = block_sum(nb, red);
        out.dmax = block_max(dmax, redf);
        out.dmin = -block_max(-dmin, redf);
    } else {
        float lm = -INFINITY;
        int bad = 0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            lm = fmaxf(lm, xq[j]);
            bad |= (xq[j] != xq[j]) || (xq[j] == INFINITY);
        }
        const float mc = block_max(lm, redf);
        double sa = 0.0;
        if (mc != -INFINITY) {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) sa += exp(((double)xq[j] - (double)mc) * invT);
        }
        out.sa = (double)mc;
        out.sb = block_sum(sa, red);
        out.pa = (double)__syncthreads_or(bad);
        out.pb = out.na = out.nb = 0.0;
        out.dmin = out.dmax = 0.0f;
    }
    if (threadIdx.x == 0) partials[(int64_t)b * nchunks + c] = out;
}

constexpr int kModeFallback = 2;  // residual of total zero: sample q itself

// Exact weight of one element of the residual: a - rho*b where q > p for
// certain, max(0, a - rho*b) in the near-threshold band, 0 below it.
__device__ __forceinline__ double residual_weight(float xq, float xp, const SeqState& s, double invT, double rho)
{
    const float d = xq - xp;
    if (!(d >= s.thr_lo)) return 0.0;
    const double a = exp(((double)xq - (double)s.mq) * invT);
    const double bb = exp(((double)xp - (double)s.mp) * invT);
    const double w = a - rho * bb;
    return (d > s.thr_hi) ? w : fmax(0.0, w);
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_sample_final(const char* __restrict__ zq, const char* __restrict__ zp,
                                                         int V, int nchunks, double invT,
                                                         const SeqState* __restrict__ st,
                                                         const ChunkSums* __restrict__ partials, int width,
                                                         int32_t* __restrict__ out_tokens,
                                                         int32_t* __restrict__ out_num,
                                                         int32_t* __restrict__ out_path,
                                                         double* __restrict__ out_resid)
{
    constexpr int EB = elem_bytes<DT>();
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const SeqState s = st[b];
    if (s.status) return;
    __shared__ double red[kWaves];
    __shared__ float redf[kWaves];
    __shared__ double s_near[kMaxChunks];
    __shared__ int s_chunk;
    __shared__ double s_base;
    __shared__ int s_owner;
    const ChunkSums* P = partials + (int64_t)b * nchunks;
    // chunks per thread (contiguous groups, token order)
    const int g = (nchunks + kBlock - 1) / kBlock;
    const int c0 = tid * g;
    const int c1 = min(nchunks, c0 + g);
    const char* qrow = zq + s.q_off * EB;
    const char* prow = zp + s.p_off * EB;

    // --- totals ---
    double rho = 0.0, M = 0.0, resid_mass = 0.0;
    int mode = s.mode;
    if (mode == kModeResidual) {
        double sq = 0.0, sp = 0.0;
        for (int c = c0; c < c1; ++c) {
            sq += P[c].sa;
            sp += P[c].sb;
        }
        sq = block_sum(sq, red);
        sp = block_sum(sp, red);
        rho = sq / sp;
        // near-threshold tokens: exact when they share one zq - zp (one ratio
        // q/p), else the chunk is rescanned below with the exact rho
        for (int c = tid; c < nchunks; c += kBlock) {
            const ChunkSums p = P[c];
            s_near[c] = (p.dmin < p.dmax) ? NAN : fmax(0.0, p.na - rho * p.nb);
        }
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            if (!(s_near[c] != s_near[c])) continue;  // uniform across the block
            float xq[kPerThread], xp[kPerThread];
            load_chunk16<DT>(qrow, V, c, tid, xq);
            load_chunk16<DT>(prow, V, c, tid, xp);
            double w = 0.0;
            for (int j = 0; j < kPerThread; ++j) {
                const float d = xq[j] - xp[j];
                if (d >= s.thr_lo && !(d > s.thr_hi)) w += residual_weight(xq[j], xp[j], s, invT, rho);
            }
            w = block_sum(w, red);
            if (tid == 0) s_near[c] = w;
            __syncthreads();
        }
        double wsum = 0.0;
        for (int c = c0; c < c1; ++c) wsum += (P[c].pa - rho * P[c].pb) + s_near[c];
        const double Wtot = block_sum(wsum, red);
        if (!(Wtot > 0.0)) {
            mode = kModeFallback;
            resid_mass = 0.0;
        } else {
            resid_mass = Wtot / sq;
        }
    } else {
        float lm = -INFINITY;
        int bad = 0;
        for (int c = c0; c < c1; ++c) {
            lm = fmaxf(lm, (float)P[c].sa);
            bad |= P[c].pa != 0.0;
        }
        M = (double)block_max(lm, redf);
        bad = __syncthreads_or(bad);
        if (bad || M == -INFINITY) {
            for (int i = tid; i < width; i += kBlock) {
                out_tokens[(int64_t)b * width + i] = -1;
                if (out_path) out_path[(int64_t)b * width + i] = -1;
            }
            if (tid == 0) out_num[b] = -1;
            return;
        }
    }
    auto chunk_weight = [&](int c) -> double {
        const ChunkSums& p = P[c];
        if (mode == kModeResidual) return (p.pa - rho * p.pb) + s_near[c];
        if (mode == kModeFallback) return p.sa;
        return (p.sa == -INFINITY) ? 0.0 : p.sb * exp((p.sa - M) * invT);
    };

    // --- locate the chunk: first chunk whose running weight exceeds u*W ---
    // The owner is the last thread whose group starts at or below the
    // threshold; it scans its group and, if rounding leaves the threshold past
    // its end, takes its last chunk of positive weight.
    double gsum = 0.0;
    for (int c = c0; c < c1; ++c) gsum += chunk_weight(c);
    double Wtot;
    const double gbase = block_exclusive_scan(gsum, red, &Wtot);
    const double target = s.u * Wtot;
    if (tid == 0) {
        s_owner = -1;
        s_chunk = 0;  // never left unset, even if no thread could claim
        s_base = 0.0;
    }
    __syncthreads();
    if (gsum > 0.0 && gbase <= target) atomicMax(&s_owner, tid);
    __syncthreads();
    if (tid == s_owner) {
        double cum = gbase;
        int pick = -1, last = -1;
        double pick_base = 0.0, last_base = 0.0;
        for (int c = c0; c < c1; ++c) {
            const double w = chunk_weight(c);
            if (w > 0.0) {
                last = c;
                last_base = cum;
                if (pick < 0 && cum + w > target) {
                    pick = c;
                    pick_base = cum;
                }
            }
            cum += w;
        }
        if (pick < 0) {
            pick = last;
            pick_base = last_base;
        }
        s_chunk = pick;
        s_base = pick_base;
    }
    __syncthreads();
    const int cs = s_chunk;
    const double cbase = s_base;

    // --- rescan the chunk ---
    float xq[kPerThread], xp[kPerThread];
    load_chunk16<DT>(qrow, V, cs, tid, xq);
    if (mode == kModeResidual) load_chunk16<DT>(prow, V, cs, tid, xp);
    double scale = 1.0, mc = 0.0;
    if (mode == kModeBonus) {
        mc = P[cs].sa;
        scale = exp((mc - M) * invT);
    }
    double w[kPerThread];
    double tsum = 0.0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        double v;
        if (mode == kModeResidual) v = residual_weight(xq[j], xp[j], s, invT, rho);
        else if (mode == kModeFallback) v = exp(((double)xq[j] - (double)s.mq) * invT);
        else v = exp(((double)xq[j] - mc) * invT);
        w[j] = v;
        tsum += v;
    }
    double ctotal;
    const double tbase = block_exclusive_scan(tsum, red, &ctotal);
    const double local = (target - cbase) / scale;
    if (tid == 0) s_owner = -1;
    __syncthreads();
    if (tsum > 0.0 && tbase <= local) atomicMax(&s_owner, tid);
    __syncthreads();
    if (s_owner < 0) {
        // no positive weight at or below the threshold in this chunk (only
        // possible through rounding): take its last element of positive weight
        int last = -1;
        for (int j = 0; j < kPerThread; ++j)
            if (w[j] > 0.0) last = cs * kChunk + tid * kPerThread + j;
        __shared__ int s_last;
        if (tid == 0) s_last = -1;
        __syncthreads();
        atomicMax(&s_last, last);
        __syncthreads();
        if (tid == 0) {
            out_tokens[(int64_t)b * width + s.k] = s_last;
            if (s_last < 0) out_num[b] = -1;
            if (out_resid) out_resid[b] = (s.mode == kModeResidual) ? resid_mass : 0.0;
        }
        return;
    }
    if (tid == s_owner) {
        double cum = tbase;
        int pick = -1, last = -1;
        for (int j = 0; j < kPerThread; ++j) {
            if (w[j] > 0.0) {
                last = j;
                if (pick < 0 && cum + w[j] > local) pick = j;
            }
            cum += w[j];
        }
        if (pick < 0) pick = last;
        out_tokens[(int64_t)b * width + s.k] = cs * kChunk + tid * kPerThread + pick;
        if (out_resid) out_resid[b] = (s.mode == kModeResidual) ? resid_mass : 0.0;
    }
}

__global__ void k_philox_uniforms(uint64_t seed, uint64_t round, int nseq, int npos, double* out_acc,
                                  double* out_samp)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)nseq * npos) return;
    const int s = (int)(i / npos), p = (int)(i - (int64_t)s * npos) + 1;
    const Words4 w = verify_block(seed, round, (uint32_t)s, (uint32_t)p);
    if (out_acc) out_acc[i] = u53(w.w0, w.w1);
    if (out_samp) out_samp[i] = u53(w.w2, w.w3);
}

}  // namespace sv

// ===========================================================================
// C ABI
// ===========================================================================
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int nchunks_of(int V) { return (V + sv::kChunk - 1) / sv::kChunk; }

struct Layout {
    size_t stats, seq, part, total;
};

Layout make_layout(int B, int rows_per_seq, int V)
{
    Layout L;
    L.stats = 0;
    L.seq = align_up((size_t)B * rows_per_seq * sizeof(sv::RowStat));
    L.part = L.seq + align_up((size_t)B * sizeof(sv::SeqState));
    L.total = L.part + align_up((size_t)B * nchunks_of(V) * sizeof(sv::ChunkSums));
    return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Rows need only be element-aligned (strides are in elements); 16-byte
// aligned rows take the all-vector path.
int check_rows(const void* base, int64_t seq_stride, int64_t row_stride, int es)
{
    if (((uintptr_t)base % (uintptr_t)es) != 0) return SV_EALIGN;
    if (seq_stride < 0 || row_stride < 0) return SV_EINVAL;
    return SV_OK;
}

int launch_status()
{
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

}  // namespace

extern "C" {

int sv_abi_version(void) { return 1; }

const char* sv_status_string(int status)
{
    switch (status) {
        case SV_OK: return "ok";
        case SV_EINVAL: return "invalid argument";
        case SV_EDTYPE: return "unsupported dtype";
        case SV_ESHAPE: return "unsupported shape";
        case SV_EALIGN: return "logits not element-aligned or KV rows not 16-byte aligned";
        case SV_EWORKSPACE: return "workspace missing or too small";
        case SV_EHIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

size_t sv_chain_workspace_bytes(int B, int N, int V)
{
    if (B < 0 || N < 0 || N > 64 || V < 1 || V > sv::kMaxChunks * sv::kChunk) return 0;
    return make_layout(B, 2 * N, V).total;
}

size_t sv_tree_workspace_bytes(int B, int T, int V)
{
    if (B < 0 || T < 0 || T + 1 > sv::kMaxNodes || V < 1 || V > sv::kMaxChunks * sv::kChunk) return 0;
    return make_layout(B, 2 * (T + 1), V).total;
}

int spec_verify_chain(const void* target_logits, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                      const void* draft_logits, int64_t drf_seq_stride, int64_t drf_row_stride, int dtype,
                      const int32_t* draft_tokens, int B, int N, int V, uint64_t seed, uint64_t round,
                      float temperature, int32_t* out_tokens, int32_t* out_num_accepted, int8_t* out_accept,
                      float* out_probs, double* out_residual_mass, void* workspace, size_t workspace_bytes,
                      const sv_timing* timing, hipStream_t stream)
{
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
    if (B < 0 || N < 0 || V < 1 || !(temperature > 0.0f) || !(temperature < INFINITY)) return SV_EINVAL;
    if (N > 64 || V > sv::kMaxChunks * sv::kChunk) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!target_logits || !out_tokens || !out_num_accepted) return SV_EINVAL;
    if (N > 0 && (!draft_logits || !draft_tokens)) return SV_EINVAL;
    const int es = dtype == SV_BF16 ? 2 : 4;
    int rc = check_rows(target_logits, tgt_seq_stride, tgt_row_stride, es);
    if (rc) return rc;
    if (N > 0 && (rc = check_rows(draft_logits, drf_seq_stride, drf_row_stride, es))) return rc;
    if ((int64_t)B * 2 * N > INT32_MAX || B > 65535) return SV_ESHAPE;
    const Layout L = make_layout(B, 2 * N, V);
    if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SV_EWORKSPACE;

    char* ws = static_cast<char*>(workspace);
    sv::RowStat* stats = reinterpret_cast<sv::RowStat*>(ws + L.stats);
    sv::SeqState* seq = reinterpret_cast<sv::SeqState*>(ws + L.seq);
    sv::ChunkSums* part = reinterpret_cast<sv::ChunkSums*>(ws + L.part);
    const char* zq = static_cast<const char*>(target_logits);
    const char* zp = static_cast<const char*>(draft_logits ? draft_logits : target_logits);
    const double invT = 1.0 / (double)temperature;
    const double cd = 1.4426950408889634074 / (double)temperature;  // log2(e) / T
    const float c = (float)cd;
    const int nch = nchunks_of(V);
    const dim3 blk(sv::kBlock);

    if (timing && timing->stats_begin && hipEventRecord(timing->stats_begin, stream) != hipSuccess) return SV_EHIP;
    if (N > 0) {
        if (dtype == SV_BF16)
            sv::k_stats_chain<sv::DT_BF16><<<dim3(B * 2 * N), blk, 0, stream>>>(
                zq, tgt_seq_stride, tgt_row_stride, zp, drf_seq_stride, drf_row_stride, N, V, c, cd, stats);
        else
            sv::k_stats_chain<sv::DT_F32><<<dim3(B * 2 * N), blk, 0, stream>>>(
                zq, tgt_seq_stride, tgt_row_stride, zp, drf_seq_stride, drf_row_stride, N, V, c, cd, stats);
        if ((rc = launch_status())) return rc;
    }
    if (timing && timing->stats_end && hipEventRecord(timing->stats_end, stream) != hipSuccess) return SV_EHIP;
    const dim3 grid_acc((B + sv::kWaves - 1) / sv::kWaves);
    if (dtype == SV_BF16)
        sv::k_accept_chain<sv::DT_BF16><<<grid_acc, blk, 0, stream>>>(
            zq, tgt_seq_stride, tgt_row_stride, zp, drf_seq_stride, drf_row_stride, draft_tokens, B, N, V, seed,
            round, invT, temperature, stats, seq, out_tokens, out_num_accepted, out_accept, out_probs);
    else
        sv::k_accept_chain<sv::DT_F32><<<grid_acc, blk, 0, stream>>>(
            zq, tgt_seq_stride, tgt_row_stride, zp, drf_seq_stride, drf_row_stride, draft_tokens, B, N, V, seed,
            round, invT, temperature, stats, seq, out_tokens, out_num_accepted, out_accept, out_probs);
    if ((rc = launch_status())) return rc;
    if (dtype == SV_BF16) {
        sv::k_sample_partials<sv::DT_BF16><<<dim3(nch, B), blk, 0, stream>>>(zq, zp, V, nch, invT, seq, part);
        sv::k_sample_final<sv::DT_BF16><<<dim3(B), blk, 0, stream>>>(zq, zp, V, nch, invT, seq, part, N + 1,
                                                                     out_tokens, out_num_accepted, nullptr,
                                                                     out_residual_mass);
    } else {
        sv::k_sample_partials<sv::DT_F32><<<dim3(nch, B), blk, 0, stream>>>(zq, zp, V, nch, invT, seq, part);
        sv::k_sample_final<sv::DT_F32><<<dim3(B), blk, 0, stream>>>(zq, zp, V, nch, invT, seq, part, N + 1,
                                                                    out_tokens, out_num_accepted, nullptr,
                                                                    out_residual_mass);
    }
    return launch_status();
}

int spec_verify_tree(const void* target_logits, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                     const void* draft_logits, int64_t drf_seq_stride, int64_t drf_row_stride, int dtype,
                     const int32_t* node_tokens, const int32_t* parents, int parents_shared, int B, int T, int V,
                     int max_depth, uint64_t seed, uint64_t round, float temperature, int32_t* out_tokens,
                     int32_t* out_path_nodes, int32_t* out_num_accepted, int8_t* out_accept, float* out_probs,
                     double* out_residual_mass, void* workspace, size_t workspace_bytes, const sv_timing* timing,
                     hipStream_t stream)
{
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
    if (B < 0 || T < 0 || V < 1 || max_depth < 0 || !(temperature > 0.0f) || !(temperature < INFINITY))
        return SV_EINVAL;
    if (T + 1 > sv::kMaxNodes || max_depth > T || V > sv::kMaxChunks * sv::kChunk) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!target_logits || !draft_logits || !node_tokens || !parents || !out_tokens || !out_path_nodes ||
        !out_num_accepted)
        return SV_EINVAL;
    const int es = dtype == SV_BF16 ? 2 : 4;
    int rc = check_rows(target_logits, tgt_seq_stride, tgt_row_stride, es);
    if (rc) return rc;
    if ((rc = check_rows(draft_logits, drf_seq_stride, drf_row_stride, es))) return rc;
    const int nn = T + 1;
    if ((int64_t)B * 2 * nn > INT32_MAX || B > 65535) return SV_ESHAPE;
    const Layout L = make_layout(B, 2 * nn, V);
    if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SV_EWORKSPACE;

    char* ws = static_cast<char*>(workspace);
    sv::RowStat* stats = reinterpret_cast<sv::RowStat*>(ws + L.stats);
    sv::SeqState* seq = reinterpret_cast<sv::SeqState*>(ws + L.seq);
    sv::ChunkSums* part = reinterpret_cast<sv::ChunkSums*>(ws + L.part);
    const char* zq = static_cast<const char*>(target_logits);
    const char* zp = static_cast<const char*>(draft_logits);
    const double invT = 1.0 / (double)temperature;
    const double cd = 1.4426950408889634074 / (double)temperature;
    const float c = (float)cd;
    const int nch = nchunks_of(V);
    const dim3 blk(sv::kBlock);

    if (timing && timing->stats_begin && hipEventRecord(timing->stats_begin, stream) != hipSuccess) return SV_EHIP;
    if (dtype == SV_BF16)
        sv::k_stats_tree<sv::DT_BF16><<<dim3(B * 2 * nn), blk, 0, stream>>>(
            zq, tgt_seq_stride, tgt_row_stride, zp, drf_seq_stride, drf_row_stride, parents, parents_shared, nn, V,
            c, cd, stats);
    else
        sv::k_stats_tree<sv::DT_F32><<<dim3(B * 2 * nn), blk, 0, stream>>>(
            zq, tgt_seq_stride, tgt_row_stride, zp, drf_seq_stride, drf_row_stride, parents, parents_shared, nn, V,
            c, cd, stats);
    if ((rc = launch_status())) return rc;
    if (timing && timing->stats_end && hipEventRecord(timing->stats_end, stream) != hipSuccess) return SV_EHIP;
    if (dtype == SV_BF16)
        sv::k_accept_tree<sv::DT_BF16><<<dim3(B), blk, 0, stream>>>(
            zq, tgt_seq_stride, tgt_row_stride, zp, drf_seq_stride, drf_row_stride, node_tokens, parents,
            parents_shared, B, T, V, max_depth, seed, round, invT, temperature, stats, seq, out_tokens,
            out_path_nodes, out_num_accepted, out_accept, out_probs);
    else
        sv::k_accept_tree<sv::DT_F32><<<dim3(B), blk, 0, stream>>>(
            zq, tgt_seq_stride, tgt_row_stride, zp, drf_seq_stride, drf_row_stride, node_tokens, parents,
            parents_shared, B, T, V, max_depth, seed, round, invT, temperature, stats, seq, out_tokens,
            out_path_nodes, out_num_accepted, out_accept, out_probs);
    if ((rc = launch_status())) return rc;
    const int width = max_depth + 1;
    if (dtype == SV_BF16) {
        sv::k_sample_partials<sv::DT_BF16><<<dim3(nch, B), blk, 0, stream>>>(zq, zp, V, nch, invT, seq, part);
        sv::k_sample_final<sv::DT_BF16><<<dim3(B), blk, 0, stream>>>(zq, zp, V, nch, invT, seq, part, width,
                                                                     out_tokens, out_num_accepted, out_path_nodes,
                                                                     out_residual_mass);
    } else {
        sv::k_sample_partials<sv::DT_F32><<<dim3(nch, B), blk, 0, stream>>>(zq, zp, V, nch, invT, seq, part);
        sv::k_sample_final<sv::DT_F32><<<dim3(B), blk, 0, stream>>>(zq, zp, V, nch, invT, seq, part, width,
                                                                    out_tokens, out_num_accepted, out_path_nodes,
                                                                    out_residual_mass);
    }
    return launch_status();
}

int sv_philox_uniforms(uint64_t seed, uint64_t round, int nseq, int npos, double* out_acc, double* out_samp,
                       hipStream_t stream)
{
    if (nseq < 0 || npos < 0) return SV_EINVAL;
    const int64_t n = (int64_t)nseq * npos;
    if (n == 0) return SV_OK;
    if (!out_acc && !out_samp) return SV_EINVAL;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > INT32_MAX) return SV_ESHAPE;
    sv::k_philox_uniforms<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(seed, round, nseq, npos, out_acc,
                                                                           out_samp);
    return launch_status();
}

}  // extern "C"
