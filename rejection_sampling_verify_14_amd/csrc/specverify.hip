// specverify.hip -- gfx950 kernel and C ABI of the verify-and-accept step
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
// Launches of one call, all on the caller's stream:
//   * Chains of bf16 logits in 16-byte aligned rows: one launch, k_chain_tab.
//     Its first blocks fill a per-call table of exp(z/T) over the bf16 grid
//     (kTabKeys); the rest form sections of 16 sequences: section k holds the
//     row blocks of sequence group k, then the accept blocks of group k - 2,
//     the chunk blocks of group k - 4 and the final-step blocks of group
//     k - 6, so the sampling of early groups runs while later groups' rows
//     stream.  Row block: the statistics (m, s), s = sum exp((z - m)/T), of
//     one ~64K-token segment of one of the 2N draft-position rows (16-byte
//     nontemporal loads, the next batch in flight; the hardware exp2 in fp32
//     with one fma per exponent argument against a wave-uniform reference,
//     summed in double).  This is the HBM-bound part.  Accept block: one
//     wave (lane i = position i+1) folds the sequence's row records, forms
//     q(d)/p(d) in the log domain in double, ballots, and stores the
//     sequence's state.  Chunk block: the sums of eight 2048-token chunks
//     (four in the last groups) of the row(s) the sequence samples from, each
//     exponential one read of the block's LDS copy of the table; the bonus
//     row is read only by sequences that sample from it.  Final block:
//     combines the chunk records, finds the chunk holding u*W, rescans it
//     with a block-wide prefix scan and writes the token (inverse CDF in
//     token order) and the KV rows.
//   * Chains of fp32 logits: the same one launch, k_chain_tab<DT_F32>,
//     without the table: its chunk blocks form the sums through a
//     table-driven fp64 exp (exp_rel).
//   * Chains of bf16 logits in rows that are not 16-byte aligned: k_rows (row
//     blocks of every row, then one accept block per sequence), then
//     k_chunks (chunk sums through exp_rel, then one final-step block per
//     sequence).
//   * Trees: k_rows (row blocks, then one tree-accept block per sequence:
//     every node tested in parallel, a wave walks the parent array with
//     ballots; the state and the walk's path go to the workspace), then
//     k_sample, whose blocks form their group of chunk sums and whose last
//     block to finish for a sequence (an arrival counter) runs the final
//     step.
// Blocks of one launch exchange data through self-validating records
// (sv_device.h): no cache-wide fences.  A block only waits for blocks of
// lower index in the same grid, which the in-order dispatch has started, and
// every wait is bounded (a wait that runs out fails the sequence with -2);
// launch boundaries carry the rest.
//
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <random>

#include "sv_device.h"
#include "specverify.h"
#include "sv_host.h"

namespace sv {

// ===========================================================================
// Pass 1: row statistics
// ===========================================================================
// Head and tail elements of a row that is not 16-byte aligned or not a whole
// number of vectors: one element at a time, against a per-lane reference.
__device__ __forceinline__ void accumulate_value(float x, float c, double cd, float& ref, double& acc)
{
    if ((x - ref) * c > 1.0f) {
        acc = (ref == -INFINITY) ? 0.0 : acc * exp2((double)(ref - x) * cd);
        ref = x;
    }
    const float r = (ref == -INFINITY) ? 0.0f : ref;
    acc += (double)__builtin_amdgcn_exp2f((x - r) * c);
}

__device__ __forceinline__ void combine_stat(float& m, double& s, float m2, double s2, double cd)
{
    const float M = fmaxf(m, m2);
    const double f1 = (m == M) ? 1.0 : exp2((double)(m - M) * cd);
    const double f2 = (m2 == M) ? 1.0 : exp2((double)(m2 - M) * cd);
    s = s * f1 + s2 * f2;
    m = M;
}

// A wave's running sum over the 16-byte vectors of a segment, against a
// reference `ref` that is the same in every lane: acc = sum 2^(x c - p) with
// p = RN(ref * c), so that each term's exponent argument is one fma; the sum
// relative to ref is acc * 2^-(ref c - p), where ref c - p (the rounding of
// the product, exact as fma(ref, c, -p)) is applied once at the end.  When
// ref * c is not a finite float (logits beyond ~2^127 T) the terms fall back
// to 2^((x - ref) c) and p = ref * c is not used.
struct WaveSum {
    float ref, p;
    double acc;
};

__device__ __forceinline__ bool wide_ref(const WaveSum& w) { return !(fabsf(w.p) < INFINITY); }

// Moves the reference up to lm (> ref), rescaling the sum.
__device__ __forceinline__ void move_ref(WaveSum& w, float lm, float c, double cd)
{
    const float np = lm * c;
    if (w.ref == -INFINITY) {
        w.acc = 0.0;
    } else if (!(fabsf(np) < INFINITY) || wide_ref(w)) {
        // leave the p form: rescale by 2^((ref - lm) c) relative to the old form's reference
        const double old = wide_ref(w) ? 1.0 : exp2(-(double)fmaf(w.ref, c, -w.p));
        w.acc *= old * exp2(((double)w.ref - (double)lm) * cd);
        if (fabsf(np) < INFINITY) w.acc *= exp2((double)fmaf(lm, c, -np));
    } else {
        w.acc *= exp2((double)w.p - (double)np);
    }
    w.ref = lm;
    w.p = np;
}

// One batch of U 16-byte vectors per lane (vectors past the end carry -inf),
// in fp32 groups of (at most) 32 terms added to the double accumulator.  When
// a group sum of any lane exceeds kGroupLimit (so a term exceeds it: an
// element more than three binary orders of magnitude, in units of the scaled
// logits, above the reference), is not finite, or comes before any reference
// exists, the reference moves to the wave's maximum of the group and the
// group is summed again; so the dominant terms keep exponent arguments below
// 3, where the fp32 rounding of the argument stays small.
constexpr float kGroupLimit = 8.0f;

template <int DT, int U>
__device__ __forceinline__ void accumulate_batch(const uint4* raw, float c, double cd, WaveSum& w)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    constexpr int GE = (U * EPV < 32) ? U * EPV : 32;  // elements per fp32 group
    constexpr int G = GE / EPV;                          // vectors per group
    static_assert(U % G == 0, "batch must hold whole groups");
#pragma unroll
    for (int g = 0; g < U / G; ++g) {
        auto group_sum = [&]() {
            float e[GE];
            if (!wide_ref(w)) {
                const float np = -w.p;
#pragma unroll
                for (int u = 0; u < G; ++u) {
                    float x[EPV];
                    decode16<DT>(raw[g * G + u], x);
#pragma unroll
                    for (int i = 0; i < EPV; ++i) e[u * EPV + i] = __builtin_amdgcn_exp2f(fmaf(x[i], c, np));
                }
            } else {
#pragma unroll
                for (int u = 0; u < G; ++u) {
                    float x[EPV];
                    decode16<DT>(raw[g * G + u], x);
#pragma unroll
                    for (int i = 0; i < EPV; ++i) e[u * EPV + i] = __builtin_amdgcn_exp2f((x[i] - w.ref) * c);
                }
            }
#pragma unroll
            for (int s = 1; s < GE; s <<= 1) {
#pragma unroll
                for (int i = 0; i + s < GE; i += 2 * s) e[i] += e[i + s];
            }
            return e[0];
        };
        auto group_max = [&]() {
            float lm = -INFINITY;
#pragma unroll
            for (int u = 0; u < G; ++u) {
                float x[EPV];
                decode16<DT>(raw[g * G + u], x);
#pragma unroll
                for (int i = 0; i < EPV; ++i) lm = fmaxf(lm, x[i]);
            }
            return wave_max(lm);
        };
        if (w.ref == -INFINITY) {
            // no reference yet (uniform across the wave): take the group maximum
            const float lm = group_max();
            if (lm != -INFINITY) move_ref(w, lm, c, cd);
        }
        float s = (w.ref == -INFINITY) ? 0.0f : group_sum();
        if (__any(!(s <= kGroupLimit))) {
            const float lm = group_max();
            if (lm > w.ref) move_ref(w, lm, c, cd);
            s = (w.ref == -INFINITY) ? 0.0f : group_sum();
        }
        w.acc += (double)s;
    }
}

// A 16-byte vector of -inf logits (pads the last batch of a row).
template <int DT>
__device__ __forceinline__ uint4 neg_inf16()
{
    const uint32_t w = (DT == DT_BF16) ? 0xff80ff80u : 0xff800000u;
    return make_uint4(w, w, w, w);
}

// Batch bt of a row's 16-byte vectors into x, U per thread, every address
// clamped into the row (a lane past the end re-reads the last vector), so
// the loads carry no branches.  nvec > 0.
template <int U>
__device__ __forceinline__ void load_batch(const uint4* __restrict__ vrow, int nvec, int bt, uint4* x)
{
    const int v0 = bt * U * kBlock + (int)threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = stream_load16(vrow + min(v0 + u * kBlock, nvec - 1));
}

// The vectors of batch bt past the row's end replaced by -inf (for the one
// partial batch, once its loads are in).
template <int DT, int U>
__device__ __forceinline__ void mask_batch(int nvec, int bt, uint4* x)
{
    const int v0 = bt * U * kBlock + (int)threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (v0 + u * kBlock >= nvec) x[u] = neg_inf16<DT>();
}

// (m, s) of n consecutive elements starting at `row`, valid in thread 0.
// Rows need only be element-aligned: the elements before the first 16-byte
// boundary are read one by one, the rest as 16-byte vectors in batches of U
// per thread, the next batch's loads issued before the current batch is used.
// The loop runs over pairs of whole batches with two register sets and an
// unconditional (clamped) prefetch: no register a load is still writing is
// copied or overwritten, and no branch merges load states, so each batch
// waits only for its own loads.  The partial batch, if any, is masked after.
// Every lane of a wave shares the reference, so the wave's sum is a plain sum
// of doubles; the four waves' (m, s) are combined by thread 0.
template <int DT, int U>
__device__ __forceinline__ RowStat block_row_stats(const char* __restrict__ row, int n, float c, double cd)
{
    constexpr int EB = elem_bytes<DT>();
    constexpr int EPV = 16 / EB;
    WaveSum w{-INFINITY, 0.0f, 0.0};
    int head = (int)(((16u - ((uint32_t)(uintptr_t)row & 15u)) & 15u) / EB);
    head = head < n ? head : n;
    // head and tail elements go to a per-lane accumulator of their own
    float ref1 = -INFINITY;
    double acc1 = 0.0;
    if ((int)threadIdx.x < head) accumulate_value(load_logit<DT>(row, threadIdx.x), c, cd, ref1, acc1);
    row += head * EB;
    n -= head;
    const int nvec = n / EPV;
    const uint4* __restrict__ vrow = reinterpret_cast<const uint4*>(row);
    const int nfull = nvec / (U * kBlock);
    const bool part = nvec > nfull * U * kBlock;
    if (nvec > 0) {
        uint4 x0[U], x1[U];
        load_batch<U>(vrow, nvec, 0, x0);
        int bt = 0;
        for (; bt + 2 <= nfull; bt += 2) {
            load_batch<U>(vrow, nvec, bt + 1, x1);
            accumulate_batch<DT, U>(x0, c, cd, w);
            load_batch<U>(vrow, nvec, bt + 2, x0);
            accumulate_batch<DT, U>(x1, c, cd, w);
        }
        // x0 holds batch bt: the last whole one, the partial one, or none
        if (bt < nfull) {
            load_batch<U>(vrow, nvec, bt + 1, x1);
            accumulate_batch<DT, U>(x0, c, cd, w);
            if (part) {
                mask_batch<DT, U>(nvec, bt + 1, x1);
                accumulate_batch<DT, U>(x1, c, cd, w);
            }
        } else if (part) {
            mask_batch<DT, U>(nvec, bt, x0);
            accumulate_batch<DT, U>(x0, c, cd, w);
        }
    }
    const int tail = n - nvec * EPV;
    if ((int)threadIdx.x < tail)
        accumulate_value(load_logit<DT>(row, (int64_t)nvec * EPV + threadIdx.x), c, cd, ref1, acc1);
    // the wave's vector sum (one reference): a plain sum, then the fma offset
    float m = w.ref;
    double s = wave_sum(w.acc);
    if (m != -INFINITY && !wide_ref(w)) s *= exp2(-(double)fmaf(w.ref, c, -w.p));
    // head and tail lanes (rare): their own (m, s), folded in
    if (__any(ref1 != -INFINITY)) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float m2 = __shfl_xor(ref1, off, 64);
            const double s2 = __shfl_xor(acc1, off, 64);
            combine_stat(ref1, acc1, m2, s2, cd);
        }
        combine_stat(m, s, ref1, acc1, cd);
    }
    __shared__ float red_m[kWaves];
    __shared__ double red_s[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
    }
    __syncthreads();
    RowStat st;
    st.m = red_m[0];
    st.s = red_s[0];
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 1; k < kWaves; ++k) combine_stat(st.m, st.s, red_m[k], red_s[k], cd);
    }
    return st;
}

__device__ __forceinline__ bool stat_bad(const RowStat& r) { return !(r.s > 0.0 && r.s < INFINITY); }

// The sum a row's statistics carry when one of its records never arrived (a
// bounded wait ran out): negative, so no row of data can have it, and bad.
constexpr double kStatTimedOut = -1.0;
__device__ __forceinline__ bool stat_timed_out(const RowStat& r) { return r.s == kStatTimedOut; }

// SeqState::status values: 0 ok, 1 data error (emitted as num_accepted =
// -1), 2 a bounded wait for another block's record ran out (emitted as -2:
// not a property of the data; never expected, since every block waited on
// has been dispatched before the waiter).
constexpr int kStatusData = 1;
constexpr int kStatusTimeout = 2;


// ===========================================================================
// Parameters of one call
// ===========================================================================
constexpr int kMaxSections = 128;  // sections of the one-launch chain step's grid

struct VerifyParams {
    const char* zq;
    const char* zp;
    int64_t qs, qr, ps, pr;   // sequence / row strides (elements)
    const int32_t* tokens;    // chain: draft tokens [B, N]; tree: node tokens [B, T+1]
    const int32_t* parents;   // tree only
    int parents_shared;
    int B, V, N, nn;          // chain: N drafts, nn = N+1; tree: nn = T+1 nodes, N unused
    int max_depth, width;     // output row width (chain N+1, tree max_depth+1)
    int walk;                 // tree: 0 first accepted child, 1 best child only
    int rows;                 // pass-1 rows per sequence (chain 2N+1, tree 2 nn)
    int segs, seg_len;        // segments per row, elements per segment
    int r_items, nch;         // row blocks per sequence (rows x segs), sample chunks per sequence
    int cpb, groups;          // sample chunks per block, sample blocks (pieces) per sequence
    uint64_t seed, round;
    float T, c;               // temperature, log2(e)/T
    double cd, invT;
    uint32_t epoch;
    int spin_limit;           // polls a wait for another block's record may take
    // exp(z/T) over the bf16 grid (bf16 logits; see kTabKeys)
    int use_tab;              // the table is filled and used
    int lazy_bonus;           // the bonus row q_N is not in the row pass: read only by a bonus sample
    int tab_blocks;           // row-kernel blocks that fill it
    uint32_t tab_lo;          // first magnitude key of the table
    // workspace
    uint64_t* chunk_arrivals; // [B] epoch-tagged arrival counters of the sample blocks
    SeqState* seqs;           // [B] accept state of each sequence (accept blocks -> sample blocks)
    int32_t* paths;           // [B][nn] trees: the walk's node path (accept blocks -> final step)
    char* stats;              // [B * rows][segs] RowStat records (row kernel -> sample kernel)
    char* part;               // [B][nch] ChunkSums records
    double* etab_g;           // [kTabEntries] the exp(z/T) table (row kernel -> sample kernels)
    char* tab_done;           // [tab_blocks] records: table block x has stored its entries
    uint32_t stats_bytes, part_bytes;
    // one-launch chain step (k_chain_tab): sequences in groups (fuse_gstart);
    // section k holds the row blocks of group k, then the accept blocks of
    // group k - fuse_la, the chunk blocks of group k - fuse_lc and the final
    // blocks of group k - fuse_lf (those that exist); sched[k] is the first
    // block of section k (after the table blocks), sched[nsec] the grid's end
    int fuse_ng, fuse_la, fuse_lc, fuse_lf, fuse_nsec;
    int sched[kMaxSections + 1];
    int fuse_gstart[kMaxSections / 2 + 1];  // group j = sequences [gstart[j], gstart[j+1])
    // chunks per chunk block and chunk blocks per sequence of each group
    // (groups whose chunk blocks come after every row block take smaller
    // ones: nothing else is left to overlap their latency with)
    int16_t fuse_cpb[kMaxSections / 2], fuse_groups[kMaxSections / 2];
    // outputs
    int32_t* out_tokens;
    int32_t* out_path;
    int32_t* out_num;
    int8_t* out_acc;
    float* out_probs;
    double* out_resid;
    const int32_t* kv_len_in;
    int32_t* out_src_rows;
    int32_t* out_kv_len;
};

// ~0.5 s of polling; never reached (every record waited for is stored by a
// block that has already finished its part)
constexpr int kSpinLimit = 1 << 19;

// Poll a record until it is this call's and whole; false after `limit`
// further polls (the call's spin_limit: kSpinLimit unless a test lowers it).
template <int K>
__device__ __forceinline__ bool wait_record(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4* a, uint32_t epoch,
                                            int limit)
{
    int spins = 0;
    while (!try_record<K>(r, off, a, epoch)) {
        if (++spins > limit) return false;
        __builtin_amdgcn_s_sleep(2);
        asm volatile("" ::: "memory");  // the next try loads again
    }
    return true;
}

// Arrival index of the caller among this call's arrivals at a counter (0 for
// the first).  A counter still carrying an earlier call's epoch is claimed
// with a compare-exchange that installs this call's epoch; after that the
// low word counts.
__device__ __forceinline__ uint32_t arrive(uint64_t* ctr, uint32_t epoch)
{
    uint64_t cur = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while ((uint32_t)(cur >> 32) != epoch) {
        const uint64_t want = ((uint64_t)epoch << 32) | 1u;
        if (__hip_atomic_compare_exchange_strong(ctr, &cur, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return 0u;
    }
    return (uint32_t)__hip_atomic_fetch_add(ctr, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stats_rsrc(const VerifyParams& P)
{
    return make_rsrc(P.stats, P.stats_bytes);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const VerifyParams& P)
{
    return make_rsrc(P.part, P.part_bytes);
}

__device__ __forceinline__ uint32_t stat_off(const VerifyParams& P, int64_t grow, int slot)
{
    return (uint32_t)((grow * P.segs + slot) * kRowStatBytes);
}

__device__ __forceinline__ uint32_t chunk_off(const VerifyParams& P, int b, int c)
{
    return (uint32_t)(((int64_t)b * P.nch + c) * kChunkSumsBytes);
}

__device__ __forceinline__ void put_chunk(const VerifyParams& P, int b, int c, const ChunkSums& v)
{
    u32x4 a[4];
    pack(v, a);
    put_record<4>(part_rsrc(P), chunk_off(P, b, c), a, P.epoch);
}

// Lane 0 stores a chunk record whose fields hold the same value in every
// lane; its tag is formed before the branch, so it stays scalar arithmetic.
__device__ __forceinline__ void put_chunk_uniform(const VerifyParams& P, int b, int c, const ChunkSums& v)
{
    u32x4 a[4];
    pack(v, a);
    a[3].w = record_tag<4>(a, P.epoch);
    if ((threadIdx.x & 63) == 0) {
        const __amdgpu_buffer_rsrc_t r = part_rsrc(P);
        const uint32_t off = chunk_off(P, b, c);
#pragma unroll
        for (int i = 0; i < 4; ++i) put_atom(r, off + 16u * i, a[i]);
    }
}

// A chunk record already known to be this call's.
__device__ __forceinline__ ChunkSums get_chunk(const VerifyParams& P, int b, int c)
{
    const __amdgpu_buffer_rsrc_t r = part_rsrc(P);
    u32x4 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = get_atom(r, chunk_off(P, b, c) + 16u * i);
    return unpack_chunk(a);
}

// Statistics of pass-1 rows from the records of their segments, kStatBatch
// segments per batch: every record of a batch is requested before any is
// used, so a batch costs one memory round trip.  A record that is not this
// call's (never expected) marks the row's result as timed out (kStatTimedOut).
constexpr int kStatBatch = 8;

// Requests the records of segments [i0, i0 + kStatBatch) of row `row` of b.
// Slots past the last segment re-read it (fold_row_stat skips them), so the
// loads carry no branches and issue back to back.
__device__ __forceinline__ void issue_row_stat(const VerifyParams& P, int b, int row, int i0, u32x4* a)
{
    const __amdgpu_buffer_rsrc_t r = stats_rsrc(P);
    const int64_t grow = (int64_t)b * P.rows + row;
#pragma unroll
    for (int j = 0; j < kStatBatch; ++j) a[j] = get_atom(r, stat_off(P, grow, min(i0 + j, P.segs - 1)));
}

// Folds the records requested by issue_row_stat into acc: the batch's
// maximum first, then each segment's sum scaled to it (independent exps, in
// segment order), then the batch into acc.  A record that is not yet this
// call's (its row block may still be running when the reader is a block of
// the same launch) is polled until it is; one that never arrives poisons the
// row's result (sum kStatTimedOut).  Past the poll the fold is branch-free.
__device__ __forceinline__ void fold_row_stat(const VerifyParams& P, int b, int row, int i0, u32x4* a,
                                              RowStat& acc, bool& ok)
{
    float xm[kStatBatch];
    double xs[kStatBatch];
    float bm = -INFINITY;
    const int64_t grow = (int64_t)b * P.rows + row;
#pragma unroll
    for (int j = 0; j < kStatBatch; ++j) {
        const bool in = i0 + j < P.segs;
        if (in && a[j].w != record_tag<1>(&a[j], P.epoch) &&
            !wait_record<1>(stats_rsrc(P), stat_off(P, grow, i0 + j), &a[j], P.epoch, P.spin_limit))
            ok = false;
        const RowStat x = unpack_rowstat(&a[j]);
        xm[j] = in ? x.m : -INFINITY;
        xs[j] = in ? x.s : 0.0;
        bm = fmaxf(bm, xm[j]);
    }
    double bs = 0.0;
#pragma unroll
    for (int j = 0; j < kStatBatch; ++j) {
        const double e = exp2((double)(xm[j] - bm) * P.cd);
        bs += xs[j] * ((xm[j] == bm) ? 1.0 : e);
    }
    if (i0 == 0) {
        acc.m = bm;
        acc.s = bs;
    } else {
        combine_stat(acc.m, acc.s, bm, bs, P.cd);
    }
}

// Statistics of R rows of sequence b, every record of a batch of each row
// requested before any is used.
template <int R>
__device__ __forceinline__ void load_row_stats(const VerifyParams& P, int b, const int* rows, RowStat* out)
{
    bool ok[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        out[q] = RowStat{0.0, -INFINITY};
        ok[q] = true;
    }
    for (int i0 = 0; i0 < P.segs; i0 += kStatBatch) {
        u32x4 a[R][kStatBatch];
#pragma unroll
        for (int q = 0; q < R; ++q) issue_row_stat(P, b, rows[q], i0, a[q]);
#pragma unroll
        for (int q = 0; q < R; ++q) fold_row_stat(P, b, rows[q], i0, a[q], out[q], ok[q]);
    }
#pragma unroll
    for (int q = 0; q < R; ++q)
        if (!ok[q]) out[q].s = kStatTimedOut;
}

template <int DT>
__device__ __forceinline__ const char* qrow_ptr(const VerifyParams& P, int b, int r)
{
    return P.zq + ((int64_t)b * P.qs + (int64_t)r * P.qr) * elem_bytes<DT>();
}

template <int DT>
__device__ __forceinline__ const char* prow_ptr(const VerifyParams& P, int b, int r)
{
    return P.zp + ((int64_t)b * P.ps + (int64_t)r * P.pr) * elem_bytes<DT>();
}

// exp((z - m)/T) over the logits of one row, m the row's reference: E(z) R
// from the bf16-grid table when the row has one (vt), else exp_rel with the
// argument as one fma, z/T - m/T.
struct ExpRow {
    double invT, mb;   // 1/T and -m/T
    lds_dptr tab;      // the block's copy of the 2^(j/N) table (see exp_rel)
    lds_dptr vt;       // the block's LDS copy of the exp(z/T) table, if tabbed (an
                       // LDS-typed pointer: reads through a generic one are
                       // flat loads, whose waits serialize; its value 0 is a
                       // valid address, so `tabbed` says whether there is one)
    double R;          // exp(-m/T), if tabbed
    double iR;         // exp(m/T) = 1/R, if tabbed
    uint32_t lo;       // the table's first magnitude key
    bool tabbed;
    // exp_rel inline: the streaming loops of rows without the table
    __device__ __forceinline__ double slow(float z) const { return exp_rel(fma((double)z, invT, mb), tab); }
    // the table where it holds z, else exp_rel (element by element; the
    // batched form is exp_batch)
    __device__ __forceinline__ double inl(float z) const
    {
        if (tabbed) {
            const int i = tab_index(z, lo);
            if (i >= 0) return vt[i] * R;
        }
        return slow(z);
    }
};

// vt: the block's LDS copy of the bf16-grid table (null for none); a row
// takes it when its reference is within kTabRefLimit of zero in units of T.
__device__ __forceinline__ ExpRow exp_row(const VerifyParams& P, double m, const double* etab, const double* vt)
{
    ExpRow e{P.invT, -m * P.invT, (lds_dptr)etab, (lds_dptr)etab, 0.0, 0.0, P.tab_lo, false};
    if (vt && fabs(e.mb) <= kTabRefLimit) {
        e.vt = (lds_dptr)vt;
        e.R = exp(e.mb);
        e.iR = exp(-e.mb);
        e.tabbed = true;
    }
    return e;
}

// ExpRow of K logits outside the streaming loops: the table reads of all K
// are issued together (one round trip, also from a global table); logits
// outside the table (the -inf past the end of a row among them) take
// exp_rel inline: a call would spill to scratch and wait on it.
template <int K>
__device__ __forceinline__ void exp_batch(const ExpRow& e, const float* z, double* out)
{
    int idx[K];
#pragma unroll
    for (int i = 0; i < K; ++i) idx[i] = e.tabbed ? tab_index(z[i], e.lo) : -1;
#pragma unroll
    for (int i = 0; i < K; ++i) out[i] = idx[i] >= 0 ? e.vt[idx[i]] : 0.0;
#pragma unroll
    for (int i = 0; i < K; ++i) out[i] = idx[i] >= 0 ? out[i] * e.R : e.slow(z[i]);
}

// ===========================================================================
// Accept
// ===========================================================================
struct AcceptOut {
    double lq, lp;  // log q(d), log p(d)
    int accepted;
};

// Accept test of one draft token from its logits zqd (verifier) and zpd
// (draft) and the two rows' statistics.
__device__ __forceinline__ AcceptOut accept_logits(float zqd, float zpd, const RowStat& rq, const RowStat& rp,
                                                   double invT, double u)
{
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

constexpr int kMaxChainN = 64;  // longest draft chain

// Chain accept of sequence b, run by one wave (lane i = position i+1), the
// only wave of its block that calls it: b's state into `out`; with
// `outputs`, also the accept flags and probabilities.
// The accept step's state of sequence b, stored by lane 0 of the calling
// wave as a tagged four-atom record (a launch that runs both the accept test
// and the sampling polls for it; later launches read it directly).
__device__ __forceinline__ void put_seq_state(const VerifyParams& P, int b, const SeqState& s)
{
    if ((threadIdx.x & 63) != 0) return;
    u32x4 a[4];
    __builtin_memcpy(a, &s, sizeof(a));
    put_record<4>(make_rsrc(P.seqs, (size_t)P.B * kSeqStateBytes), (uint32_t)b * kSeqStateBytes, a, P.epoch);
}

// Sequence b's state once its record has landed (bounded wait), as
// wave-uniform values (lane 0's copy: every lane polled the same whole
// record), so what depends on it stays scalar; a state that never arrives
// reads as a timeout of the sequence.
__device__ __forceinline__ SeqState wait_seq_state(const VerifyParams& P, int b)
{
    u32x4 a[4];
    const bool ok = wait_record<4>(make_rsrc(P.seqs, (size_t)P.B * kSeqStateBytes), (uint32_t)b * kSeqStateBytes, a,
                                   P.epoch, P.spin_limit);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[4 * i + 0] = __builtin_amdgcn_readfirstlane(a[i].x);
        w[4 * i + 1] = __builtin_amdgcn_readfirstlane(a[i].y);
        w[4 * i + 2] = __builtin_amdgcn_readfirstlane(a[i].z);
        w[4 * i + 3] = __builtin_amdgcn_readfirstlane(a[i].w);
    }
    SeqState s;
    __builtin_memcpy(&s, w, sizeof(w));
    if (!__all(ok)) {
        s = SeqState{};
        s.status = kStatusTimeout;
    }
    return s;
}

template <int DT>
__device__ __forceinline__ void chain_accept(const VerifyParams& P, int b, RowStat* s_rows, bool outputs)
{
    const int lane = threadIdx.x;
    const int N = P.N;
    const bool active = lane < N;
    int err = 0, acc = 1;
    // every independent load first: the token, then (with the token's
    // logits in flight) the records of the 2N+1 pass-1 rows, lane j folding
    // row j (and j + 64 ...), so each lane combines one row's segments
    const int tok = active ? P.tokens[(int64_t)b * N + lane] : 0;
    const bool tok_ok = tok >= 0 && tok < P.V;
    float zqd = 0.0f, zpd = 0.0f;
    if (active && tok_ok) {
        zqd = load_logit<DT>(qrow_ptr<DT>(P, b, lane), tok);
        zpd = load_logit<DT>(prow_ptr<DT>(P, b, lane), tok);
    }
    for (int r0 = 0; r0 < P.rows; r0 += 64) {
        const int row = min(r0 + lane, P.rows - 1);
        RowStat st{0.0, -INFINITY};
        if (!(P.lazy_bonus && row == N)) load_row_stats<1>(P, b, &row, &st);
        if (r0 + lane < P.rows) s_rows[row] = st;
    }
    // one wave runs this: its LDS stores are published to its own lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the bonus row's statistics (used if all accept) and those of q_i, p_i
    const RowStat qn = s_rows[N];
    const RowStat rq = s_rows[active ? lane : N], rp = s_rows[active ? N + 1 + lane : N];
    int tmo = 0;
    if (active) {
        if (!tok_ok || stat_bad(rq) || stat_bad(rp)) {
            err = 1;
            tmo = stat_timed_out(rq) || stat_timed_out(rp);
        } else {
            const double u = accept_uniform(P.seed, P.round, (uint32_t)b, (uint32_t)(lane + 1));
            const AcceptOut o = accept_logits(zqd, zpd, rq, rp, P.invT, u);
            acc = o.accepted;
            if (outputs && P.out_probs) {
                P.out_probs[((int64_t)b * N + lane) * 2 + 0] = (float)exp(o.lq);
                P.out_probs[((int64_t)b * N + lane) * 2 + 1] = (float)exp(o.lp);
            }
        }
    }
    const uint64_t errmask = __ballot(err);
    const uint64_t rejmask = __ballot(active && !acc);
    SeqState s{};
    if (errmask) {
        s.status = __ballot(tmo) ? kStatusTimeout : kStatusData;
        put_seq_state(P, b, s);
        return;
    }
    const int k = rejmask ? (__ffsll((unsigned long long)rejmask) - 1) : N;
    if (outputs && active && P.out_acc) P.out_acc[(int64_t)b * N + lane] = (int8_t)acc;
    // statistics of row k (residual) travel from lane k
    RowStat kq, kp;
    const int src = k < N ? k : 0;
    kq.m = __shfl(rq.m, src, 64);
    kq.s = __shfl(rq.s, src, 64);
    kp.m = __shfl(rp.m, src, 64);
    kp.s = __shfl(rp.s, src, 64);
    s.k = k;
    s.node = k;
    s.status = 0;
    s.u = sample_uniform(P.seed, P.round, (uint32_t)b, (uint32_t)(k + 1));
    if (k < N) {
        fill_residual_state(s, kq, kp, P.T);
    } else {
        s.mode = kModeBonus;
        if (P.lazy_bonus) {
            // the bonus row has no row statistics: its chunks are summed in
            // units of exp(z/T) (reference 0) and the sampler checks it
            s.mq = 0.0f;
            s.bonus_ref = 0;
        } else if (stat_bad(qn)) {
            // NaN, +inf or no mass in the bonus row (or its records timed out)
            s.status = stat_timed_out(qn) ? kStatusTimeout : kStatusData;
        } else {
            s.mq = qn.m;
            s.bonus_ref = 1;
        }
    }
    put_seq_state(P, b, s);
}

constexpr int kMaxNodes = 1024;
// Nodes below this index keep their rows' statistics in LDS from the node
// tests (the walk's residual step reads them there).
constexpr int kStatCacheNodes = 64;

// Tree accept of sequence b, run by the whole block: every node n >= 1 is
// tested against its parent's q/p rows, then wave 0 walks from the root into
// the lowest-index accepted child (walk 0), or into the lowest-index child
// while it is accepted (walk 1, the pages' literal best-child walk).  The state goes to `out` and the path to
// `path` (both LDS); with `outputs`, also the accept flags and probabilities.
template <int DT>
__device__ __forceinline__ void tree_accept(const VerifyParams& P, int b, SeqState& out, int32_t* path, bool outputs)
{
    const int nn = P.nn;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int s_par[kMaxNodes];
    __shared__ unsigned char s_acc[kMaxNodes];
    __shared__ unsigned char s_kids[kMaxNodes];
    __shared__ RowStat s_pst[kStatCacheNodes][2];
    const int32_t* par = P.parents_shared ? P.parents : P.parents + (int64_t)b * nn;
    const int32_t* tok = P.tokens + (int64_t)b * nn;
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
            if (t < 0 || t >= P.V) err = 1;
        }
    }
    err = __syncthreads_or(err);
    if (!err) {
        for (int n = 1 + tid; n < nn; n += kBlock) {
            const int p = s_par[n];
            const int t = tok[n];
            const float zqd = load_logit<DT>(qrow_ptr<DT>(P, b, p), t);
            const float zpd = load_logit<DT>(prow_ptr<DT>(P, b, p), t);
            const int rows[2] = {2 * p, 2 * p + 1};
            RowStat st[2];
            load_row_stats<2>(P, b, rows, st);
            const RowStat rq = st[0], rp = st[1];
            if (stat_bad(rq) || stat_bad(rp)) {
                err |= (stat_timed_out(rq) || stat_timed_out(rp)) ? 2 : 1;
                continue;
            }
            if (p < kStatCacheNodes) {
                // every child of p stores the same two values
                s_pst[p][0] = rq;
                s_pst[p][1] = rp;
            }
            const double u = accept_uniform(P.seed, P.round, (uint32_t)b, (uint32_t)n);
            const AcceptOut o = accept_logits(zqd, zpd, rq, rp, P.invT, u);
            s_acc[n] = (unsigned char)o.accepted;
            if (outputs && P.out_acc) P.out_acc[(int64_t)b * nn + n] = (int8_t)o.accepted;
            if (outputs && P.out_probs) {
                P.out_probs[((int64_t)b * nn + n) * 2 + 0] = (float)exp(o.lq);
                P.out_probs[((int64_t)b * nn + n) * 2 + 1] = (float)exp(o.lp);
            }
        }
    }
    const int tmo = __syncthreads_or(err & 2);  // (a predicate: the timeout bit first)
    err = __syncthreads_or(err);
    SeqState s{};
    if (err) {
        s.status = tmo ? kStatusTimeout : kStatusData;
        if (tid == 0) out = s;
        return;
    }
    if (tid == 0 && outputs) {
        if (P.out_acc) P.out_acc[(int64_t)b * nn] = 1;
        if (P.out_probs) {
            P.out_probs[(int64_t)b * nn * 2 + 0] = 0.0f;
            P.out_probs[(int64_t)b * nn * 2 + 1] = 0.0f;
        }
    }
    if (wave != 0) return;
    if (lane == 0) path[0] = 0;
    int cur = 0, depth = 0, residual = 0, werr = 0;
    for (;;) {
        if (!s_kids[cur]) break;  // leaf: bonus from q at cur
        int next = -1;
        for (int base = cur + 1; base < nn; base += 64) {
            const int n = base + lane;
            const bool pred = n < nn && s_par[n] == cur && (P.walk == 1 || s_acc[n]);
            const uint64_t m = __ballot(pred);
            if (m) {
                next = base + __ffsll((unsigned long long)m) - 1;
                break;
            }
        }
        // walk 1: the best child decides alone (its rejection ends the walk)
        if (next >= 0 && P.walk == 1 && !s_acc[next]) next = -1;
        if (next < 0) {
            residual = 1;
            break;
        }
        if (depth + 1 > P.max_depth) {
            werr = 1;
            break;
        }
        ++depth;
        if (lane == 0) path[depth] = next;
        cur = next;
    }
    if (werr) {
        s.status = kStatusData;
    } else {
        s.k = depth;
        s.node = cur;
        s.status = 0;
        s.u = sample_uniform(P.seed, P.round, (uint32_t)b, (uint32_t)(depth + 1));
        if (residual) {
            RowStat st[2];
            if (cur < kStatCacheNodes) {
                // stored by cur's children's tests (every one passed)
                st[0] = s_pst[cur][0];
                st[1] = s_pst[cur][1];
            } else {
                const int rows[2] = {2 * cur, 2 * cur + 1};
                load_row_stats<2>(P, b, rows, st);
            }
            fill_residual_state(s, st[0], st[1], P.T);
            // (read and checked by the node tests above; a record that
            // vanished since would be a timeout)
            if (stat_bad(st[0]) || stat_bad(st[1])) s.status = kStatusTimeout;
        } else {
            s.mode = kModeBonus;
        }
    }
    if (lane == 0) out = s;
}

// ===========================================================================
// Sampling
// ===========================================================================
// The kPerThread elements of thread `tid` in chunk `c` (contiguous, token
// order); entries past V read as -inf.
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
        // unconditional loads (past V, of the chunk's first token), then -inf
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t e = e0 + j;
            const float v = load_logit<DT>(row, e < V ? e : (int64_t)c * kChunk);
            x[j] = e < V ? v : -INFINITY;
        }
    }
}

constexpr int kModeFallback = 2;  // residual of total zero: sample q itself

// Rows a sequence samples from, with the row index clamped into range (the
// clamp keeps any index in bounds whatever the state holds).
template <int DT>
__device__ __forceinline__ const char* sample_qrow(const VerifyParams& P, int b, const SeqState& s)
{
    const int node = min(max(s.node, 0), P.nn - 1);
    return qrow_ptr<DT>(P, b, node);
}

template <int DT>
__device__ __forceinline__ const char* sample_prow(const VerifyParams& P, int b, const SeqState& s)
{
    const int lim = (P.parents ? P.nn : P.N) - 1;
    const int node = min(max(s.node, 0), max(lim, 0));
    return prow_ptr<DT>(P, b, node);
}

// A wave's view of a chunk: lane `lane` owns the 16-byte vectors
// lane + 64*k, k < kChunk / (64 * elements per vector), so each load
// instruction of the wave reads 1 KB of consecutive bytes.  Rows that are
// 16-byte aligned with V a whole number of vectors are read as vectors, each
// wholly inside the row or wholly past V (then -inf, chunk_vec_tail); other
// rows token by token.
template <int DT>
__device__ __forceinline__ bool row_vectors(const char* row, int V)
{
    return (((uintptr_t)row) & 15u) == 0 && V % (16 / elem_bytes<DT>()) == 0;
}

// Whether chunk c ends at or before V (every chunk but possibly the last).
__device__ __forceinline__ bool chunk_whole(int V, int c)
{
    return (int64_t)(c + 1) * kChunk <= V;
}

#ifndef SV_LANE_AHEAD
#define SV_LANE_AHEAD 2
#endif
#ifndef SV_BONUS_AHEAD
#define SV_BONUS_AHEAD 4
#endif
// 16-byte vectors per row a lane keeps in flight: two rows of residual
// steps, or one row of the shorter bonus steps
constexpr int kLaneAhead = SV_LANE_AHEAD;
constexpr int kBonusAhead = SV_BONUS_AHEAD;
// the table path's vectors in flight per row (two ran faster than four on
// B=256 N=7 V=128256 bf16 chains)
#ifndef SV_TAB_AHEAD
#define SV_TAB_AHEAD 2
#endif
constexpr int kTabAhead = SV_TAB_AHEAD;
#ifndef SV_STEP_BARRIER
#define SV_STEP_BARRIER 1
#endif
#ifndef SV_CHUNK_WAVES
#define SV_CHUNK_WAVES 4
#endif

// The lane's k-th vector of chunk c.
template <int DT>
__device__ __forceinline__ uint4 chunk_vec(const char* __restrict__ row, int c, int k, int lane)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    return reinterpret_cast<const uint4*>(row)[(int64_t)c * (kChunk / EPV) + 64 * k + lane];
}

// Token t of the lane's share in the element-by-element path (chunk c <
// nch); past V an unconditional load of the chunk's first token, then -inf.
template <int DT>
__device__ __forceinline__ float chunk_token(const char* row, int V, int c, int lane, int k, int i)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    const int64_t e = (int64_t)c * kChunk + (int64_t)(lane + 64 * k) * EPV + i;
    const float x = load_logit<DT>(row, e < V ? e : (int64_t)c * kChunk);
    return e < V ? x : -INFINITY;
}

// The lane's k-th vector of chunk c (c < nch) of a row that row_vectors
// admits, -inf past V.  The load is unconditional (past V it re-reads the
// chunk's first vector, which lies inside the row) and the select comes
// after: a load under a branch would be waited for at the branch's end.
template <int DT>
__device__ __forceinline__ uint4 chunk_vec_tail(const char* __restrict__ row, int V, int c, int k, int lane)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    const int64_t e0 = (int64_t)c * kChunk + (int64_t)(64 * k + lane) * EPV;
    const bool in = e0 < V;
    const uint4 v = chunk_vec<DT>(row, c, in ? k : 0, in ? lane : 0);
    const uint32_t ninf = DT == DT_BF16 ? 0xFF80FF80u : 0xFF800000u;
    return in ? v : make_uint4(ninf, ninf, ninf, ninf);
}

// The lane's k-th vector of chunk c, decoded, for any row (vec: the row
// passes row_vectors).
template <int DT>
__device__ __forceinline__ void chunk_elems(const char* row, bool vec, int V, int c, int k, int lane, float* x)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    if (vec) {
        decode16<DT>(chunk_vec_tail<DT>(row, V, c, k, lane), x);
    } else {
#pragma unroll
        for (int i = 0; i < EPV; ++i) x[i] = chunk_token<DT>(row, V, c, lane, k, i);
    }
}

// ExpRow of K logits: TAB, the table's batched reads (exp_batch); else
// exp_rel inline (kernels that never take the table).
template <int K, bool TAB>
__device__ __forceinline__ void exp_vec(const ExpRow& e, const float* x, double* out)
{
    if constexpr (TAB) {
        exp_batch<K>(e, x, out);
    } else {
#pragma unroll
        for (int i = 0; i < K; ++i) out[i] = e.slow(x[i]);
    }
}

// Centre and widened half-width of the near-threshold band [thr_lo, thr_hi]
// as a test |d - mid| <= hw that every d in the band passes despite the
// rounding of d - mid; tokens it admits beyond the band only trigger
// near_chunk, whose own test is the exact one.
struct NearBand {
    float mid, hw;
};

__device__ __forceinline__ NearBand near_band(const SeqState& s)
{
    const float mid = 0.5f * s.thr_lo + 0.5f * s.thr_hi;
    const float hw = (0.5f * s.thr_hi - 0.5f * s.thr_lo) * 1.001f + fabsf(mid) * 0x1.0p-20f + 0x1.0p-100f;
    return {mid, hw};
}

// The residual's all-token and certain-region sums (sa sb pa pb of
// ChunkSums) over K token pairs; nd tracks the smallest |d - mid| (see
// NearBand), so a lane saw a near-threshold token iff nd <= hw.
template <int K, bool TAB>
__device__ __forceinline__ void residual_vec(const float* zq, const float* zp, const SeqState& s,
                                             const NearBand& nb, const ExpRow& eq, const ExpRow& ep,
                                             double* acc, float& nd)
{
    double a[K], bb[K];
    exp_vec<K, TAB>(eq, zq, a);
    exp_vec<K, TAB>(ep, zp, bb);
#pragma unroll
    for (int i = 0; i < K; ++i) {
        acc[0] += a[i];
        acc[1] += bb[i];
        const float d = zq[i] - zp[i];
        // a 0/1 factor: fma with 1 adds exactly, with 0 leaves the sum
        const double fa = d > s.thr_hi ? 1.0 : 0.0;
        acc[2] = fma(fa, a[i], acc[2]);
        acc[3] = fma(fa, bb[i], acc[3]);
        nd = fminf(nd, fabsf(d - nb.mid));  // NaN d leaves nd
    }
}

// Near-threshold band of chunk c (na nb dmin dmax of ChunkSums), element by
// element in the lane order of the vector loops, so each lane's sums equal
// those the fused loop would form.  Taken only when a wave saw a near token
// in the chunk (none in most chunks).
template <int DT, bool TAB>
__device__ __forceinline__ void near_chunk(const VerifyParams& P, const SeqState& s, const char* qrow,
                                           const char* prow, int c, const ExpRow& eq, const ExpRow& ep,
                                           ChunkSums& out)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    constexpr int PER = kChunk / EPV / 64;
    // vectors per row loaded together: the chunk's loads of a group are all
    // in flight before the first is used (one memory round trip per group)
    constexpr int G = PER < 4 ? PER : 4;
    static_assert(PER % G == 0, "whole groups of vectors");
    const int lane = threadIdx.x & 63;
    const bool vec = row_vectors<DT>(qrow, P.V) && row_vectors<DT>(prow, P.V);
    double na = 0.0, nb = 0.0;
    float dmin = INFINITY, dmax = -INFINITY;
    auto add = [&](const float* xq, const float* xp) {
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            const float d = xq[i] - xp[i];
            if (d >= s.thr_lo && !(d > s.thr_hi)) {
                na += TAB ? eq.inl(xq[i]) : eq.slow(xq[i]);
                nb += TAB ? ep.inl(xp[i]) : ep.slow(xp[i]);
                dmin = fminf(dmin, d);
                dmax = fmaxf(dmax, d);
            }
        }
    };
    if (vec) {
#pragma unroll 1
        for (int k0 = 0; k0 < PER; k0 += G) {
            uint4 vq[G], vp[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                vq[j] = chunk_vec_tail<DT>(qrow, P.V, c, k0 + j, lane);
                vp[j] = chunk_vec_tail<DT>(prow, P.V, c, k0 + j, lane);
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float xq[EPV], xp[EPV];
                decode16<DT>(vq[j], xq);
                decode16<DT>(vp[j], xp);
                add(xq, xp);
            }
        }
    } else {
#pragma unroll 1
        for (int k = 0; k < PER; ++k) {
            float xq[EPV], xp[EPV];
            chunk_elems<DT>(qrow, false, P.V, c, k, lane, xq);
            chunk_elems<DT>(prow, false, P.V, c, k, lane, xp);
            add(xq, xp);
        }
    }
    out.na = wave_sum(na);
    out.nb = wave_sum(nb);
    out.dmax = wave_max(dmax);
    out.dmin = -wave_max(-dmin);
}

// The residual's sums over chunk c by one wave (see residual_vec); returns
// whether the wave saw a near-threshold token.  Vector rows: every load of
// the chunk issued first, then one vector at a time.
template <int DT, bool TAB>
__device__ __forceinline__ bool residual_chunk(const VerifyParams& P, const SeqState& s, const char* qrow,
                                               const char* prow, int c, const ExpRow& eq, const ExpRow& ep,
                                               double* acc)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    constexpr int PER = kChunk / EPV / 64;  // vectors per lane: bf16 4, fp32 8
    const int lane = threadIdx.x & 63;
    const NearBand nb = near_band(s);
    float nd = INFINITY;
    if (row_vectors<DT>(qrow, P.V) && row_vectors<DT>(prow, P.V)) {
        uint4 vq[PER], vp[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            vq[k] = chunk_vec_tail<DT>(qrow, P.V, c, k, lane);
            vp[k] = chunk_vec_tail<DT>(prow, P.V, c, k, lane);
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            float xq[EPV], xp[EPV];
            decode16<DT>(vq[k], xq);
            decode16<DT>(vp[k], xp);
            residual_vec<EPV, TAB>(xq, xp, s, nb, eq, ep, acc, nd);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll 1
        for (int k = 0; k < PER; ++k) {
            float xq[EPV], xp[EPV];
            chunk_elems<DT>(qrow, false, P.V, c, k, lane, xq);
            chunk_elems<DT>(prow, false, P.V, c, k, lane, xp);
            residual_vec<EPV, TAB>(xq, xp, s, nb, eq, ep, acc, nd);
        }
    }
    return nd <= nb.hw;
}

// Maximum and NaN/+inf flag of the lane's tokens of a chunk.
template <int DT>
__device__ __forceinline__ void bonus_max(const VerifyParams& P, const char* qrow, int c, float& lm, int& bad)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    constexpr int PER = kChunk / EPV / 64;
    const int lane = threadIdx.x & 63;
    auto take = [&](const float* x) {
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            lm = fmaxf(lm, x[i]);
            bad |= (x[i] != x[i]) || (x[i] == INFINITY);
        }
    };
    if (row_vectors<DT>(qrow, P.V)) {
        uint4 v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) v[k] = chunk_vec_tail<DT>(qrow, P.V, c, k, lane);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            float x[EPV];
            decode16<DT>(v[k], x);
            take(x);
        }
    } else {
#pragma unroll 1
        for (int k = 0; k < PER; ++k) {
            float x[EPV];
            chunk_elems<DT>(qrow, false, P.V, c, k, lane, x);
            take(x);
        }
    }
}

template <int DT, bool TAB>
__device__ __forceinline__ double bonus_sum(const VerifyParams& P, const char* qrow, int c, const ExpRow& ec)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    constexpr int PER = kChunk / EPV / 64;
    const int lane = threadIdx.x & 63;
    double sa = 0.0;
    auto add = [&](const float* x) {
        double a[EPV];
        exp_vec<EPV, TAB>(ec, x, a);
#pragma unroll
        for (int i = 0; i < EPV; ++i) sa += a[i];
    };
    if (row_vectors<DT>(qrow, P.V)) {
        uint4 v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) v[k] = chunk_vec_tail<DT>(qrow, P.V, c, k, lane);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            float x[EPV];
            decode16<DT>(v[k], x);
            add(x);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll 1
        for (int k = 0; k < PER; ++k) {
            float x[EPV];
            chunk_elems<DT>(qrow, false, P.V, c, k, lane, x);
            add(x);
        }
    }
    return sa;
}

// Chunk sums of the whole chunks [ca, cb) of 16-byte aligned rows, by one
// wave, stored as records, through exp_rel.  BONUS: the q row alone, summed
// against its pass-1 reference s.mq; otherwise the residual's sums over the
// q and p rows.  The loop runs over whole chunks with the chunk's vectors
// unrolled: D slots per row, slot k % D refilled with the vector D ahead
// (clamped to the range's last), and no exit inside a chunk, so the slots
// keep their registers and each vector waits only for its own loads.
template <int DT, bool BONUS>
__device__ __forceinline__ void chunk_range(const VerifyParams& P, int b, const SeqState& s, const char* qrow, const char* prow,
                            int ca, int cb, const ExpRow& eq, const ExpRow& ep)
{
    constexpr int EPV = 16 / elem_bytes<DT>();
    constexpr int PER = kChunk / EPV / 64;  // vectors per lane per chunk: bf16 4, fp32 8
    constexpr int D = BONUS ? kBonusAhead : kLaneAhead;
    static_assert(PER % D == 0, "slots rotate within a chunk");
    const int lane = threadIdx.x & 63;
    const int nvec = (cb - ca) * PER;
    if (nvec <= 0) return;
    const uint4* vq = reinterpret_cast<const uint4*>(qrow) + (int64_t)ca * (kChunk / EPV) + lane;
    const uint4* vp = reinterpret_cast<const uint4*>(prow) + (int64_t)ca * (kChunk / EPV) + lane;
    uint4 sq[D], sp[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(j, nvec - 1);
        sq[j] = vq[64 * t];
        sp[j] = BONUS ? sq[j] : vp[64 * t];
    }
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    const NearBand nb = near_band(s);
    float nd = INFINITY;
#pragma unroll 1
    for (int c = ca; c < cb; ++c) {
        const int t0 = (c - ca) * PER;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int j = k % D;
            float xq[EPV], xp[EPV];
            decode16<DT>(sq[j], xq);
            if constexpr (!BONUS) decode16<DT>(sp[j], xp);
            const int tn = min(t0 + k + D, nvec - 1);
            sq[j] = vq[64 * tn];
            if constexpr (!BONUS) sp[j] = vp[64 * tn];
            if constexpr (BONUS) {
                double a[EPV];
                exp_vec<EPV, false>(eq, xq, a);
#pragma unroll
                for (int i = 0; i < EPV; ++i) acc[0] += a[i];
            } else {
                residual_vec<EPV, false>(xq, xp, s, nb, eq, ep, acc, nd);
            }
            // the sums are formed here, vector by vector
            asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(nd));
#if SV_STEP_BARRIER
            __builtin_amdgcn_sched_barrier(0);  // one vector's work at a time
#endif
        }
        ChunkSums out{};
        if constexpr (BONUS) {
            out.sa = (double)s.mq;
            out.sb = wave_sum(acc[0]);
        } else {
            out.sa = wave_sum(acc[0]);
            out.sb = wave_sum(acc[1]);
            out.pa = wave_sum(acc[2]);
            out.pb = wave_sum(acc[3]);
            out.dmin = INFINITY;
            out.dmax = -INFINITY;
            if (__ballot(nd <= nb.hw)) near_chunk<DT, false>(P, s, qrow, prow, c, eq, ep, out);
            nd = INFINITY;
        }
        if (lane == 0) put_chunk(P, b, c, out);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = 0.0;
    }
}

// Sums of one wave over a chunk of the table path.
struct TabSums {
    double acc[4];  // sa sb pa pb in units of exp(z/T)
    float nd;       // smallest |d - mid| seen (see NearBand)
    // bonus rows (summed with no row statistics): the logits outside the
    // table, per lane against the largest of them, oref: oacc = sum of
    // exp((z - oref)/T); obad: a NaN or +inf logit
    float oref;
    double oacc;
    int obad;
};

__device__ __forceinline__ void tab_sums_clear(TabSums& A)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) A.acc[i] = 0.0;
    A.nd = INFINITY;
    A.oref = -INFINITY;
    A.oacc = 0.0;
    A.obad = 0;
}

// A bonus-row logit outside the table into the lane's running sum against
// its own largest such logit (rescaled when a larger one comes).
__device__ __forceinline__ void bonus_outside(float z, const ExpRow& e, TabSums& A)
{
    if (!(z == z) || z == INFINITY) {
        A.obad = 1;
    } else if (z > -INFINITY) {
        if (z > A.oref) {
            if (A.oref > -INFINITY) A.oacc *= exp_rel(((double)A.oref - (double)z) * e.invT, e.tab);
            A.oref = z;
        }
        A.oacc += exp_rel(((double)z - (double)A.oref) * e.invT, e.tab);
    }
}

// The chunk record of a bonus row from a wave's table sums: the reference is
// the larger of 0 (the units of the table sums) and the largest logit
// outside the table, sb the chunk's sum of exp((z - reference)/T); a chunk
// without mass gets reference -inf.  Fields wave-uniform.
__device__ __forceinline__ void bonus_record(const TabSums& A, const ExpRow& e, ChunkSums& out)
{
    const double sin = lane_value(wave_sum(A.acc[0]), 0);
    double ref = 0.0, sb = sin;
    if (__ballot(A.oref > -INFINITY)) {
        const float mo = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(wave_max(A.oref))));
        ref = fmax(0.0, (double)mo);
        const double own = A.oref > -INFINITY ? A.oacc * exp_rel(((double)A.oref - ref) * e.invT, e.tab) : 0.0;
        sb = sin * exp_rel(-ref * e.invT, e.tab) + lane_value(wave_sum(own), 0);
    }
    out.sa = sb > 0.0 ? ref : -INFINITY;
    out.sb = sb;
    out.flags = __ballot(A.obad) ? kFlagBad : 0u;
}

// One 16-byte vector per row (8 token pairs, or 8 tokens of the q row alone
// for BONUS) into the sums: 16 table reads issued together, then the terms;
// a ballot sends a vector with a logit outside the table to the rare path,
// one element per trip.
template <bool BONUS>
__device__ __forceinline__ void tab_vector(const uint4 vq, const uint4 vp, const SeqState& s, const NearBand& nb,
                                           const ExpRow& eq, const ExpRow& ep, uint32_t lo, lds_cptr tab,
                                           TabSums& A)
{
    const uint32_t wq[4] = {vq.x, vq.y, vq.z, vq.w};
    const uint32_t wp[4] = {vp.x, vp.y, vp.z, vp.w};
    const u16x2 lo2 = {(unsigned short)lo, (unsigned short)lo};
    u16x2 worst = {0, 0};
    // two halves of four token pairs: eight table reads in flight, then
    // their terms (the halves keep the live table values to 16 registers)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        double e[4], f[4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int k = 2 * h + kk;
            uint32_t a0, a1;
            tab_offsets(wq[k], lo2, a0, a1, worst);
            e[2 * kk] = lds_f64(tab, a0);
            e[2 * kk + 1] = lds_f64(tab, a1);
            if constexpr (!BONUS) {
                tab_offsets(wp[k], lo2, a0, a1, worst);
                f[2 * kk] = lds_f64(tab, a0);
                f[2 * kk + 1] = lds_f64(tab, a1);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = 4 * h + j;
            if constexpr (BONUS) {
                A.acc[0] += e[j];
            } else {
                const float zq = (i & 1) ? bf16_hi(wq[i >> 1]) : bf16_lo(wq[i >> 1]);
                const float zp = (i & 1) ? bf16_hi(wp[i >> 1]) : bf16_lo(wp[i >> 1]);
                const float d = zq - zp;
                const double fa = d > s.thr_hi ? 1.0 : 0.0;
                A.acc[0] += e[j];
                A.acc[1] += f[j];
                A.acc[2] = fma(fa, e[j], A.acc[2]);
                A.acc[3] = fma(fa, f[j], A.acc[3]);
                A.nd = fminf(A.nd, fabsf(d - nb.mid));
            }
        }
        asm volatile("" : "+v"(A.acc[0]), "+v"(A.acc[1]), "+v"(A.acc[2]), "+v"(A.acc[3]), "+v"(A.nd));
    }
    if (__any(max((uint32_t)worst.x, (uint32_t)worst.y) >= (uint32_t)kTabKeys)) {
        // logits outside the table: their terms went in as zeros.  One
        // element per trip, its word chosen by selects (a rolled loop keeps
        // the rare path's registers few).
#pragma unroll 1
        for (int i = 0; i < 8; ++i) {
            const int k = i >> 1;
            const uint32_t w = k == 0 ? wq[0] : k == 1 ? wq[1] : k == 2 ? wq[2] : wq[3];
            const float zq = (i & 1) ? bf16_hi(w) : bf16_lo(w);
            const bool oq = tab_index(zq, lo) < 0;
            // exp((z - m)/T) / R = exp(z/T): into the table values' units
            if constexpr (BONUS) {
                if (oq) bonus_outside(zq, eq, A);
            } else {
                const uint32_t v = k == 0 ? wp[0] : k == 1 ? wp[1] : k == 2 ? wp[2] : wp[3];
                const float zp = (i & 1) ? bf16_hi(v) : bf16_lo(v);
                const bool op = tab_index(zp, lo) < 0;
                const double fa = (zq - zp > s.thr_hi) ? 1.0 : 0.0;
                // -inf adds exactly zero (the padding past V of a partial
                // chunk is -inf): skipped; NaN still goes through exp_rel,
                // whose NaN reaches the sums
                if (oq && zq != -INFINITY) {
                    const double a = eq.slow(zq) * eq.iR;
                    A.acc[0] += a;
                    A.acc[2] = fma(fa, a, A.acc[2]);
                }
                if (op && zp != -INFINITY) {
                    const double bb = ep.slow(zp) * ep.iR;
                    A.acc[1] += bb;
                    A.acc[3] = fma(fa, bb, A.acc[3]);
                }
            }
        }
    }
}

// chunk_range for 16-byte aligned bf16 rows with the bf16-grid table in LDS
// (tab; see kTabKeys): each exponential is one table read.  The lane sums of
// table values are in units of exp(z/T) and are scaled by the row's R once
// per chunk; logits outside the table (none in most vectors) are added
// through exp_rel, in units of exp((z - m)/T), to sums of their own.  Both
// rows must have the table (eq.tabbed, and ep.tabbed unless BONUS).  The loop runs
// over whole chunks with the chunk's vectors unrolled: D slots per row, slot
// k % D refilled with the vector D ahead (clamped to the range's last), and
// no exit inside a chunk, so the slots keep their registers.
// The first kTabAhead vectors per row of chunks [ca, cb) of the calling
// lane (a range's loads in flight before the table is in LDS).
struct TabSlots {
    uint4 q[kTabAhead], p[kTabAhead];
};

template <bool BONUS>
__device__ __forceinline__ void tab_first_loads(const char* qrow, const char* prow, int ca, int cb, TabSlots& sl)
{
    constexpr int PER = kChunk / 8 / 64;
    const int lane = threadIdx.x & 63;
    const int nvec = (cb - ca) * PER;
    if (nvec <= 0) return;  // no range: chunk_range_tab loads nothing either
    const uint4* vq = reinterpret_cast<const uint4*>(qrow) + (int64_t)ca * (kChunk / 8) + lane;
    const uint4* vp = reinterpret_cast<const uint4*>(prow) + (int64_t)ca * (kChunk / 8) + lane;
#pragma unroll
    for (int j = 0; j < kTabAhead; ++j) {
        const int t = min(j, nvec - 1);
        sl.q[j] = vq[64 * t];
        sl.p[j] = BONUS ? sl.q[j] : vp[64 * t];
    }
}

template <bool BONUS>
__device__ __forceinline__ void chunk_range_tab(const VerifyParams& P, int b, const SeqState& s, const char* qrow, const char* prow,
                                int ca, int cb, const ExpRow& eq, const ExpRow& ep, lds_cptr tab, TabSlots& sl)
{
    constexpr int PER = kChunk / 8 / 64;  // vectors per lane per chunk
    constexpr int D = kTabAhead;
    static_assert(PER % D == 0, "slots rotate within a chunk");
    const int lane = threadIdx.x & 63;
    const int nvec = (cb - ca) * PER;
    if (nvec <= 0) return;
    const uint4* vq = reinterpret_cast<const uint4*>(qrow) + (int64_t)ca * (kChunk / 8) + lane;
    const uint4* vp = reinterpret_cast<const uint4*>(prow) + (int64_t)ca * (kChunk / 8) + lane;
    uint4 (&sq)[D] = sl.q;
    uint4 (&sp)[D] = sl.p;
    const NearBand nb = near_band(s);
    TabSums A;
    tab_sums_clear(A);
#pragma unroll 1
    for (int c = ca; c < cb; ++c) {
        const int t0 = (c - ca) * PER;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int j = k % D;
            const uint4 xq = sq[j], xp = sp[j];
            const int tn = min(t0 + k + D, nvec - 1);
            sq[j] = vq[64 * tn];
            if constexpr (!BONUS) sp[j] = vp[64 * tn];
            tab_vector<BONUS>(xq, xp, s, nb, eq, ep, P.tab_lo, tab, A);
            // the sums are formed here, vector by vector: without this the
            // compiler may defer the additions to the chunk's end and keep
            // every table value of the chunk in registers
            asm volatile("" : "+v"(A.acc[0]), "+v"(A.acc[1]), "+v"(A.acc[2]), "+v"(A.acc[3]), "+v"(A.nd));
#if SV_STEP_BARRIER
            __builtin_amdgcn_sched_barrier(0);
#endif
        }
        // the chunk's record: sums made wave-uniform, so its tag is
        // computed by scalar instructions
        ChunkSums out{};
        if constexpr (BONUS) {
            bonus_record(A, eq, out);
        } else {
            double t[4];
            wave_sum4(eq.R * A.acc[0], ep.R * A.acc[1], eq.R * A.acc[2], ep.R * A.acc[3], t);
            out.sa = t[0];
            out.sb = t[1];
            out.pa = t[2];
            out.pb = t[3];
            out.dmin = INFINITY;
            out.dmax = -INFINITY;
            if (__ballot(A.nd <= nb.hw)) {
                near_chunk<DT_BF16, true>(P, s, qrow, prow, c, eq, ep, out);
                // equal in every lane already: taken from lane 0 as scalars
                out.na = lane_value(out.na, 0);
                out.nb = lane_value(out.nb, 0);
                out.dmin = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(out.dmin)));
                out.dmax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(out.dmax)));
            }
            A.nd = INFINITY;
        }
        put_chunk_uniform(P, b, c, out);
        tab_sums_clear(A);
    }
}

// One chunk c of 16-byte aligned bf16 rows from the LDS table, by one wave,
// with every vector of the chunk loaded at once (one memory round trip): the
// partial last chunk, whose vectors past V read as -inf (their keys lie
// outside the table and add exp_rel(-inf) = 0).  tab_chunk_load issues the
// loads, tab_chunk_sums forms and stores the record.
struct TabChunk {
    uint4 q[kChunk / 8 / 64], p[kChunk / 8 / 64];
};

template <bool BONUS>
__device__ __forceinline__ void tab_chunk_load(const VerifyParams& P, const char* qrow, const char* prow, int c,
                                               TabChunk& ch)
{
    constexpr int PER = kChunk / 8 / 64;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        ch.q[k] = chunk_vec_tail<DT_BF16>(qrow, P.V, c, k, lane);
        ch.p[k] = BONUS ? ch.q[k] : chunk_vec_tail<DT_BF16>(prow, P.V, c, k, lane);
    }
}

template <bool BONUS>
__device__ __forceinline__ void tab_chunk_sums(const VerifyParams& P, int b, const SeqState& s, const char* qrow, const char* prow,
                               int c, const ExpRow& eq, const ExpRow& ep, lds_cptr tab, const TabChunk& ch)
{
    constexpr int PER = kChunk / 8 / 64;
    const NearBand nb = near_band(s);
    TabSums A;
    tab_sums_clear(A);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        tab_vector<BONUS>(ch.q[k], ch.p[k], s, nb, eq, ep, P.tab_lo, tab, A);
        asm volatile("" : "+v"(A.acc[0]), "+v"(A.acc[1]), "+v"(A.acc[2]), "+v"(A.acc[3]), "+v"(A.nd));
        __builtin_amdgcn_sched_barrier(0);
    }
    ChunkSums out{};
    if constexpr (BONUS) {
        bonus_record(A, eq, out);
    } else {
        double t[4];
        wave_sum4(eq.R * A.acc[0], ep.R * A.acc[1], eq.R * A.acc[2], ep.R * A.acc[3], t);
        out.sa = t[0];
        out.sb = t[1];
        out.pa = t[2];
        out.pb = t[3];
        out.dmin = INFINITY;
        out.dmax = -INFINITY;
        if (__ballot(A.nd <= nb.hw)) {
            near_chunk<DT_BF16, true>(P, s, qrow, prow, c, eq, ep, out);
            out.na = lane_value(out.na, 0);
            out.nb = lane_value(out.nb, 0);
            out.dmin = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(out.dmin)));
            out.dmax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(out.dmax)));
        }
    }
    put_chunk_uniform(P, b, c, out);
}

template <bool BONUS>
__device__ __forceinline__ void partial_chunk_tab(const VerifyParams& P, int b, const SeqState& s, const char* qrow,
                                  const char* prow, int c, const ExpRow& eq, const ExpRow& ep, lds_cptr tab)
{
    TabChunk ch;
    tab_chunk_load<BONUS>(P, qrow, prow, c, ch);
    tab_chunk_sums<BONUS>(P, b, s, qrow, prow, c, eq, ep, tab, ch);
}

// Chunk sums of the row(s) a sequence samples from (see ChunkSums), by one
// wave; valid in every lane.
template <int DT, bool TAB>
__device__ __forceinline__ ChunkSums wave_chunk_sums(const VerifyParams& P, const SeqState& s, const char* qrow, const char* prow,
                                     int c, const ExpRow& eq, const ExpRow& ep, const double* etab,
                                     const double* vt)
{
    ChunkSums out{};
    if (s.mode == kModeResidual) {
        double acc[4] = {0.0, 0.0, 0.0, 0.0};  // sa sb pa pb
        const bool near = residual_chunk<DT, TAB>(P, s, qrow, prow, c, eq, ep, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = wave_sum(acc[i]);
        out.sa = acc[0];
        out.sb = acc[1];
        out.pa = acc[2];
        out.pb = acc[3];
        out.dmin = INFINITY;
        out.dmax = -INFINITY;
        if (__ballot(near)) near_chunk<DT, TAB>(P, s, qrow, prow, c, eq, ep, out);
    } else if (s.bonus_ref) {
        // against the row's pass-1 reference (its NaN/+inf check is the
        // pass-1 statistics')
        const double sa = bonus_sum<DT, TAB>(P, qrow, c, eq);
        out.sa = (double)s.mq;
        out.sb = wave_sum(sa);
    } else {
        // the chunk maximum first, then the sum relative to it
        float lm = -INFINITY;
        int bad = 0;
        bonus_max<DT>(P, qrow, c, lm, bad);
        const float mc = wave_max(lm);
        double sa = 0.0;
        if (mc != -INFINITY) sa = bonus_sum<DT, TAB>(P, qrow, c, exp_row(P, mc, etab, vt));
        out.sa = (double)mc;
        out.sb = wave_sum(sa);
        out.flags = __any(bad) ? kFlagBad : 0u;
    }
    return out;
}

// Exact weight of one element of the residual: a - rho*b where q > p for
// certain, max(0, a - rho*b) in the near-threshold band, 0 below it.
__device__ __forceinline__ double residual_weight_of(float xq, float xp, const SeqState& s, double a, double bb,
                                                     double rho)
{
    const float d = xq - xp;
    if (!(d >= s.thr_lo)) return 0.0;
    const double w = a - rho * bb;
    return (d > s.thr_hi) ? w : fmax(0.0, w);
}

template <bool TAB>
__device__ __forceinline__ double residual_weight(float xq, float xp, const SeqState& s, const ExpRow& eq,
                                                  const ExpRow& ep, double rho)
{
    const float d = xq - xp;
    if (!(d >= s.thr_lo)) return 0.0;
    return residual_weight_of(xq, xp, s, TAB ? eq.inl(xq) : eq.slow(xq), TAB ? ep.inl(xp) : ep.slow(xp), rho);
}

// Block-wide: every output slot of sequence b that does not depend on the
// sampled token: slots i < k hold the accepted tokens, slots past k -1, and
// (trees) the path up to depth k.  emit_sample then writes slot k, the count
// and the residual mass; a failure rewrites everything through emit.
template <bool TREE>
__device__ __forceinline__ void emit_accepted(const VerifyParams& P, int b, int k, const int32_t* path)
{
    const int width = P.width;
    for (int i = threadIdx.x; i < width; i += kBlock) {
        int32_t t = -1, pn = -1;
        if (TREE) {
            if (i <= k) pn = path[i];
            if (i < k) {
                const int node = path[i + 1];
                t = P.tokens[(int64_t)b * P.nn + min(max(node, 0), P.nn - 1)];
            }
        } else if (i < k) {
            t = P.tokens[(int64_t)b * P.N + i];
        }
        if (i != k) P.out_tokens[(int64_t)b * width + i] = t;
        if (TREE) P.out_path[(int64_t)b * width + i] = pn;
        if (P.out_src_rows) {
            const int node = TREE ? pn : (i <= k ? i : -1);
            P.out_src_rows[(int64_t)b * width + i] = node >= 0 ? P.kv_len_in[b] + node : -1;
        }
    }
    if (threadIdx.x == 0 && P.out_kv_len) P.out_kv_len[b] = P.kv_len_in[b] + k + 1;
}

// Block-wide: the outputs of sequence b.  k < 0 or token < 0 marks the
// sequence as failed (every slot -1).
template <bool TREE>
__device__ __forceinline__ void emit(const VerifyParams& P, int b, int k, int token, double resid, const int32_t* path)
{
    const int width = P.width;
    const bool ok = k >= 0 && token >= 0;
    for (int i = threadIdx.x; i < width; i += kBlock) {
        int32_t t = -1, pn = -1;
        if (ok) {
            if (TREE) {
                if (i <= k) pn = path[i];
                if (i < k) {
                    const int node = path[i + 1];
                    t = P.tokens[(int64_t)b * P.nn + min(max(node, 0), P.nn - 1)];
                }
            } else if (i < k) {
                t = P.tokens[(int64_t)b * P.N + i];
            }
            if (i == k) t = token;
        }
        P.out_tokens[(int64_t)b * width + i] = t;
        if (TREE) P.out_path[(int64_t)b * width + i] = pn;
        if (P.out_src_rows) {
            const int node = !ok ? -1 : TREE ? pn : (i <= k ? i : -1);
            P.out_src_rows[(int64_t)b * width + i] = node >= 0 ? P.kv_len_in[b] + node : -1;
        }
    }
    if (threadIdx.x == 0) {
        P.out_num[b] = ok ? k : (k == -2 ? -2 : -1);
        if (P.out_resid) P.out_resid[b] = ok ? resid : 0.0;
        // the KV cache keeps the pending token and the k accepted drafts; a
        // failed sequence keeps its length
        if (P.out_kv_len) P.out_kv_len[b] = P.kv_len_in[b] + (ok ? k + 1 : 0);
    }
}

// One thread: the sampled slot of a sequence whose other slots emit_accepted
// wrote.
__device__ __forceinline__ void emit_sample(const VerifyParams& P, int b, int k, int token, double resid)
{
    P.out_tokens[(int64_t)b * P.width + k] = token;
    P.out_num[b] = k;
    if (P.out_resid) P.out_resid[b] = resid;
}

// Chunk records the final step keeps in LDS.
constexpr int kFinalCache = 256;
// Chunk records per lane of wave 0 whose loads are issued together.
constexpr int kFinalLaneBatch = 4;

// What wave 0 of the final step hands the block.
struct FinalPlan {
    double rho, M, sq, cbase, target, resid;
    int mode, cs, near_any, fail;
};

// Final step of sequence b: its chunk records, totals, chunk location,
// rescan of that chunk, outputs.  Wave 0 alone reads the records (lane L
// owns chunks [L*g, L*g + g), g = ceil(nch / 64)), forms the totals and
// locates the chunk with wave scans and ballots, and hands the block a plan
// through one barrier; the block then rescans the chunk.
// s_cs and s_near are LDS arrays of the caller (kFinalCache records and
// kMaxChunks doubles); vt is the bf16-grid table or null.
template <int DT, bool TREE, bool TAB>
__device__ __forceinline__ void sample_final(const VerifyParams& P, int b, const SeqState& s, const int32_t* path,
                             const double* etab, ChunkSums* s_cs, double* s_near, const double* vt)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nchunks = P.nch;
    const double invT = P.invT;
    __shared__ double red[kWaves];
    __shared__ FinalPlan s_plan;
    __shared__ int s_cand[kWaves];
    __shared__ int s_token;
    // the chunk records are kept in s_cs (the first kFinalCache of them;
    // later ones are read again when needed)
    if (s.status) {
        emit<TREE>(P, b, s.status == kStatusTimeout ? -2 : -1, -1, 0.0, path);
        return;
    }
    const int k = s.k;
    emit_accepted<TREE>(P, b, k, path);
    if (tid == 0) s_token = -1;
    auto chunk_at = [&](int c) -> ChunkSums { return c < kFinalCache ? s_cs[c] : get_chunk(P, b, c); };
    const char* qrow = sample_qrow<DT>(P, b, s);
    const char* prow = s.mode == kModeResidual ? sample_prow<DT>(P, b, s) : qrow;
    const ExpRow eq = exp_row(P, s.mq, etab, vt), ep = exp_row(P, s.mp, etab, vt);

    // --- wave 0: records, totals, location ---
    const int g = (nchunks + 63) / 64;
    const int c0 = lane * g, c1 = min(nchunks, c0 + g);
    int mode = s.mode;
    double rho = 0.0, M = 0.0, sq = 0.0;
    bool near_any = false;
    auto chunk_weight = [&](int c) -> double {
        const ChunkSums p = chunk_at(c);
        if (mode == kModeResidual) return (p.pa - rho * p.pb) + (near_any ? s_near[c] : 0.0);
        if (mode == kModeFallback) return p.sa;
        return (p.sa == -INFINITY) ? 0.0 : p.sb * exp((p.sa - M) * invT);
    };
    // the first chunk whose running weight exceeds u*W: its owner is the
    // last lane whose group starts at or below the threshold; it scans its
    // group and, if rounding leaves the threshold past its end, takes its
    // last chunk of positive weight
    auto locate = [&]() {
        double gsum = 0.0;
        for (int c = c0; c < c1; ++c) gsum += chunk_weight(c);
        double Wtot, gbase = wave_exclusive_scan(gsum, &Wtot);
        double resid = 0.0;
        if (mode == kModeResidual) {
            // the residual's mass; none (q <= p everywhere) falls back to q
            if (Wtot > 0.0) {
                resid = Wtot / sq;
            } else {
                mode = kModeFallback;
                gsum = 0.0;
                for (int c = c0; c < c1; ++c) gsum += chunk_weight(c);
                gbase = wave_exclusive_scan(gsum, &Wtot);
            }
        }
        const double target = s.u * Wtot;
        const uint64_t cand = __ballot(gsum > 0.0 && gbase <= target);
        const int owner = cand ? 63 - __clzll((long long)cand) : -1;
        if (lane == 0) {
            s_plan.mode = mode;
            s_plan.resid = resid;
            s_plan.target = target;
            s_plan.cs = 0;  // never left unset, even if no lane could claim
            s_plan.cbase = 0.0;
        }
        if (lane == owner) {
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
            s_plan.cs = pick < 0 ? 0 : pick;
            s_plan.cbase = pick_base;
        }
    };
    if (wave == 0) {
        int ok = 1, bad = 0;
        double sums[3] = {0.0, 0.0, 0.0};  // sa, sb, chunks with near tokens
        float lm = -INFINITY;
        auto take = [&](int c, const ChunkSums& v) {
            if (c < kFinalCache) s_cs[c] = v;
            if (mode == kModeResidual) {
                sums[0] += v.sa;
                sums[1] += v.sb;
                sums[2] += (v.na != 0.0 || v.nb != 0.0 || v.dmin <= v.dmax) ? 1.0 : 0.0;
            } else {
                lm = fmaxf(lm, (float)v.sa);
                bad |= (v.flags & kFlagBad) != 0;
            }
        };
        const __amdgpu_buffer_rsrc_t r = part_rsrc(P);
        // the first kFinalLaneBatch records of the lane requested together
        u32x4 a[kFinalLaneBatch][4];
#pragma unroll
        for (int j = 0; j < kFinalLaneBatch; ++j)
            if (c0 + j < c1)
#pragma unroll
                for (int i = 0; i < 4; ++i) a[j][i] = get_atom(r, chunk_off(P, b, c0 + j) + 16u * i);
#pragma unroll
        for (int j = 0; j < kFinalLaneBatch; ++j)
            if (c0 + j < c1) {
                if (a[j][3].w == record_tag<4>(a[j], P.epoch) ||
                    wait_record<4>(r, chunk_off(P, b, c0 + j), a[j], P.epoch, P.spin_limit))
                    take(c0 + j, unpack_chunk(a[j]));
                else
                    ok = 0;
            }
        for (int c = c0 + kFinalLaneBatch; c < c1; ++c) {
            u32x4 x[4];
            if (wait_record<4>(r, chunk_off(P, b, c), x, P.epoch, P.spin_limit)) take(c, unpack_chunk(x));
            else ok = 0;
        }
        // 2: a chunk record never arrived (timeout); 1: a data error
        int fail = !__all(ok) ? 2 : 0;
        if (!fail) {
            if (mode == kModeResidual) {
#pragma unroll
                for (int i = 0; i < 3; ++i) sums[i] = wave_sum(sums[i]);
                sq = sums[0];
                rho = sums[0] / sums[1];
                near_any = sums[2] > 0.0;
            } else {
                M = (double)wave_max(lm);
                fail = (__any(bad) || M == -INFINITY) ? 1 : 0;
            }
        }
        if (!fail && !near_any) locate();
        if (lane == 0) {
            s_plan.fail = fail;
            s_plan.near_any = near_any;
            s_plan.rho = rho;
            s_plan.M = M;
            s_plan.sq = sq;
        }
    }
    __syncthreads();
    if (s_plan.fail) {
        emit<TREE>(P, b, s_plan.fail == 2 ? -2 : -1, -1, 0.0, path);
        return;
    }
    rho = s_plan.rho;
    M = s_plan.M;
    sq = s_plan.sq;
    near_any = s_plan.near_any != 0;
    if (near_any) {
        // near-threshold tokens (rare): exact when they share one zq - zp
        // (one ratio q/p), else the chunk is rescanned with the exact rho
        for (int c = tid; c < nchunks; c += kBlock) {
            const ChunkSums p = chunk_at(c);
            s_near[c] = (p.dmin < p.dmax) ? NAN : fmax(0.0, p.na - rho * p.nb);
        }
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            if (!(s_near[c] != s_near[c])) continue;  // uniform across the block
            float xq[kPerThread], xp[kPerThread];
            load_chunk16<DT>(qrow, P.V, c, tid, xq);
            load_chunk16<DT>(prow, P.V, c, tid, xp);
            double w[1] = {0.0};
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) {
                const float d = xq[j] - xp[j];
                if (d >= s.thr_lo && !(d > s.thr_hi)) w[0] += residual_weight<TAB>(xq[j], xp[j], s, eq, ep, rho);
            }
            block_sum_n<1>(w, red);
            if (tid == 0) s_near[c] = w[0];
            __syncthreads();
        }
        if (wave == 0) locate();
        __syncthreads();
    }
    mode = s_plan.mode;
    const int cs = s_plan.cs;
    const double cbase = s_plan.cbase, target = s_plan.target, resid = s_plan.resid;

    // --- rescan the chunk: each thread its 8 tokens, from registers ---
    float xq[kPerThread], xp[kPerThread];
    load_chunk16<DT>(qrow, P.V, cs, tid, xq);
    if (mode == kModeResidual) load_chunk16<DT>(prow, P.V, cs, tid, xp);
    double scale = 1.0, mc = 0.0;
    if (mode == kModeBonus) {
        mc = chunk_at(cs).sa;
        scale = exp((mc - M) * invT);
    }
    const ExpRow ec = exp_row(P, mc, etab, vt);
    double wv[kPerThread];
    if (mode == kModeResidual) {
        double av[kPerThread], bv[kPerThread];
        exp_vec<kPerThread, TAB>(eq, xq, av);
        exp_vec<kPerThread, TAB>(ep, xp, bv);
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) wv[j] = residual_weight_of(xq[j], xp[j], s, av[j], bv[j], rho);
    } else {
        exp_vec<kPerThread, TAB>(mode == kModeFallback ? eq : ec, xq, wv);
    }
    double tsum = 0.0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) tsum += wv[j];
    double ctotal;
    const double tbase = block_exclusive_scan(tsum, red, &ctotal);
    const double local = (target - cbase) / scale;
    // the owner is the last thread whose tokens start at or below the
    // threshold: per-wave candidates by ballot, then the highest wave's
    const uint64_t cand = __ballot(tsum > 0.0 && tbase <= local);
    if (lane == 0) s_cand[wave] = cand ? wave * 64 + 63 - __clzll((long long)cand) : -1;
    __syncthreads();
    int owner = -1;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) owner = max(owner, s_cand[w]);
    const double rmass = (s.mode == kModeResidual) ? resid : 0.0;
    if (owner >= 0) {
        if (tid == owner) {
            double cum = tbase;
            int pick = -1, last = -1;
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) {
                const double wj = wv[j];
                if (wj > 0.0) {
                    last = j;
                    if (pick < 0 && cum + wj > local) pick = j;
                }
                cum += wj;
            }
            if (pick < 0) pick = last;
            emit_sample(P, b, k, cs * kChunk + tid * kPerThread + pick, rmass);
        }
        return;
    }
    // no positive weight at or below the threshold in this chunk (only
    // possible through rounding): take its last element of positive weight
    int last = -1;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
        if (wv[j] > 0.0) last = cs * kChunk + tid * kPerThread + j;
    atomicMax(&s_token, last);
    __syncthreads();
    if (s_token >= 0) {
        if (tid == 0) emit_sample(P, b, k, s_token, rmass);
    } else {
        emit<TREE>(P, b, -1, -1, 0.0, path);
    }
}

// ===========================================================================
// Kernels
// ===========================================================================
// Entries x * kBlock + threadIdx.x of the bf16-grid table (see kTabKeys).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t etab_rsrc(const VerifyParams& P)
{
    return make_rsrc(P.etab_g, (uint32_t)(kTabEntries * sizeof(double)));
}

// Table block x stores entries [x*kBlock, (x+1)*kBlock) with agent-coherent
// stores, waits until they have landed, and then stores its done record, so
// a block of the same launch that has seen every done record reads the
// whole table with coherent loads.
__device__ __forceinline__ void fill_value_table(const VerifyParams& P, int x)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const int i = x * kBlock + (int)threadIdx.x;
    if (i < kTabEntries) {
        const int sgn = i >= kTabHalf ? 1 : 0;
        const int t = i - sgn * kTabHalf;
        double v = 0.0;
        if (t < kTabKeys) {
            const uint32_t key = (P.tab_lo + (uint32_t)t) | ((uint32_t)sgn << 15);
            v = exp((double)__uint_as_float(key << 16) / (double)P.T);
        }
        const uint64_t w = (uint64_t)__double_as_longlong(v);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{(uint32_t)w, (uint32_t)(w >> 32)}, etab_rsrc(P),
                                              i * (int)sizeof(double), 0, kCpolSc1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        u32x4 a[1] = {u32x4{(uint32_t)x, 0x7ab1e000u, 0u, 0u}};
        put_record<1>(make_rsrc(P.tab_done, (uint32_t)(P.tab_blocks * 16)), (uint32_t)x * 16u, a, P.epoch);
    }
}

// Every table block's done record (wave 0 polls, the block waits at the
// barrier); false if one never arrived.
__device__ __forceinline__ bool wait_value_table(const VerifyParams& P)
{
    __shared__ int s_ok;
    if (threadIdx.x < 64) {
        int ok = 1;
        for (int x = (int)threadIdx.x; x < P.tab_blocks; x += 64) {
            u32x4 a[1];
            ok &= wait_record<1>(make_rsrc(P.tab_done, (uint32_t)(P.tab_blocks * 16)), (uint32_t)x * 16u, a,
                                 P.epoch, P.spin_limit)
                      ? 1
                      : 0;
        }
        ok = __all(ok);
        if (threadIdx.x == 0) s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

// The block's LDS copy of the table through coherent loads (the table was
// stored in this launch): every load issued before the first LDS store.
__device__ __forceinline__ void copy_value_table_coherent(const VerifyParams& P, double* pool)
{
    constexpr int N2 = kTabEntries / 2;
    constexpr int PER = (N2 + kBlock - 1) / kBlock;
    const __amdgpu_buffer_rsrc_t r = etab_rsrc(P);
    u32x4 v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = (int)threadIdx.x + k * kBlock;
        v[k] = get_atom(r, (uint32_t)(i < N2 ? i : N2 - 1) * 16u);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(pool);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = (int)threadIdx.x + k * kBlock;
        if (i < N2) dst[i] = v[k];
    }
}

// The block's LDS copy of the table (publish it with a barrier): every load
// is issued before the first LDS store, so the copy costs one round trip.
__device__ __forceinline__ void copy_value_table(const VerifyParams& P, double* pool)
{
    constexpr int N2 = kTabEntries / 2;
    constexpr int PER = (N2 + kBlock - 1) / kBlock;
    const double2* src = reinterpret_cast<const double2*>(P.etab_g);
    double2* dst = reinterpret_cast<double2*>(pool);
    double2 v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = (int)threadIdx.x + k * kBlock;
        v[k] = src[i < N2 ? i : N2 - 1];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = (int)threadIdx.x + k * kBlock;
        if (i < N2) dst[i] = v[k];
    }
}

// The final step's LDS arrays, carved from one pool: kFinalCache chunk
// records, then kMaxChunks doubles.
constexpr int kFinalPoolDoubles = (int)(kFinalCache * sizeof(ChunkSums) / sizeof(double));
constexpr int kFinalPool = kFinalPoolDoubles + kMaxChunks;
static_assert(kTabEntries % 2 == 0, "table copied as double2");

// Chunk sums of chunks [c, cb) of sequence b by the calling wave through
// exp_rel: whole chunks of aligned rows in one streaming range, the rest
// chunk by chunk.
template <int DT>
__device__ __forceinline__ void wave_chunks(const VerifyParams& P, int b, const SeqState& s, const char* qrow,
                                            const char* prow, int c, int cb, const ExpRow& eq, const ExpRow& ep,
                                            const double* etab)
{
    if (s.status == 0 && (s.mode == kModeResidual || s.bonus_ref) &&
        ((((uintptr_t)qrow) | ((uintptr_t)prow)) & 15u) == 0) {
        const int whole = min(cb, P.V / kChunk);
        if (whole > c) {
            if (s.mode == kModeResidual) chunk_range<DT, false>(P, b, s, qrow, prow, c, whole, eq, ep);
            else chunk_range<DT, true>(P, b, s, qrow, prow, c, whole, eq, ep);
            c = whole;
        }
    }
    for (; c < cb; ++c) {
        ChunkSums out{};
        if (s.status == 0) out = wave_chunk_sums<DT, false>(P, s, qrow, prow, c, eq, ep, etab, nullptr);
        if ((threadIdx.x & 63) == 0) put_chunk(P, b, c, out);
    }
}

// 16-byte loads per thread per batch of a row block
#ifndef SV_ROW_BATCH
#define SV_ROW_BATCH 4
#endif
constexpr int kRowBatch = SV_ROW_BATCH;
// Row kernel: block (b, row, segment) streams one segment of a pass-1 row
// and stores its (m, s) record.  Then come the blocks that fill the bf16-grid
// table (bf16 logits) and, for chains, B blocks of one accept test each.  Chains: rows 0..N are q rows 0..N (row N
// the bonus row) and rows N+1..2N the p rows 0..N-1.  Trees: row 2n is node
// n's q row and 2n+1 its p row, streamed only for nodes that have a child
// (an accept test reads them; the others get a placeholder record).  Many small blocks, dispatched as
// compute units free up, balance the stream better than a resident grid
// with fixed shares.
// Row block (b, idx): idx = row * segs + segment; streams the segment and
// stores its (m, s) record.
template <int DT, bool TREE>
__device__ __forceinline__ void row_block(const VerifyParams& P, int b, int idx)
{
    int row = idx / P.segs;
    const int seg = idx - row * P.segs;
    if (!TREE && P.lazy_bonus && row >= P.N) ++row;  // rows 0..N-1 (q), then N+1..2N (p)
    const char* base;
    bool work = true;
    if constexpr (TREE) {
        const int node = row >> 1;
        const int32_t* par = P.parents_shared ? P.parents : P.parents + (int64_t)b * P.nn;
        int found = 0;
        for (int m = node + 1 + (int)threadIdx.x; m < P.nn; m += kBlock) found |= (par[m] == node);
        work = __syncthreads_or(found) != 0;
        base = (row & 1) ? prow_ptr<DT>(P, b, node) : qrow_ptr<DT>(P, b, node);
    } else {
        base = row <= P.N ? qrow_ptr<DT>(P, b, row) : prow_ptr<DT>(P, b, row - P.N - 1);
    }
    RowStat st{0.0, -INFINITY};
    if (work) {
        const int begin = seg * P.seg_len;
        const int n = min(P.V - begin, P.seg_len);
        st = block_row_stats<DT, kRowBatch>(base + (int64_t)begin * elem_bytes<DT>(), n, P.c, P.cd);
    }
    if (threadIdx.x == 0) {
        u32x4 a[1];
        pack(st, a);
        put_record<1>(stats_rsrc(P), stat_off(P, (int64_t)b * P.rows + row, seg), a, P.epoch);
    }
}

template <int DT, bool TREE>
__global__ __launch_bounds__(kBlock) void k_rows(const VerifyParams P)
{
    const int nrow_blocks = P.B * P.r_items;
    if ((int)blockIdx.x >= nrow_blocks) {
        const int x = (int)blockIdx.x - nrow_blocks;
        if (x < P.tab_blocks) {
            fill_value_table(P, x);
            return;
        }
        // the accept test of sequence x - tab_blocks (chains: by wave 0;
        // trees: the whole block, then the state and the walk's path go to
        // the workspace).  Blocks are dispatched in index order, so every
        // row block has started when this one does; it polls b's records as
        // they land.
        const int b = x - P.tab_blocks;
        if constexpr (TREE) {
            __shared__ SeqState s_state;
            __shared__ int32_t s_path[kMaxNodes];
            tree_accept<DT>(P, b, s_state, s_path, true);
            __syncthreads();
            const SeqState st = s_state;
            if (threadIdx.x < 64) put_seq_state(P, b, st);
            if (st.status == 0)
                for (int i = (int)threadIdx.x; i <= st.k; i += kBlock) P.paths[(int64_t)b * P.nn + i] = s_path[i];
        } else {
            if (threadIdx.x >= 64) return;
            __shared__ RowStat s_rows[2 * kMaxChainN + 1];
            chain_accept<DT>(P, b, s_rows, true);
        }
        return;
    }
    const int b = (int)blockIdx.x / P.r_items;
    row_block<DT, TREE>(P, b, (int)blockIdx.x - b * P.r_items);
}


// ---------------------------------------------------------------------------
// Chain sample step
// ---------------------------------------------------------------------------
// The accept tests ran at the end of the row launch; this launch forms the
// chunk sums (many blocks per sequence, where the arithmetic is) and ends
// with the final step (one block per sequence).

// Blocks [0, B*groups): block (b, g) forms the chunk sums of group g of
// sequence b's chunks, one contiguous share per wave, stored as records.
// Blocks [B*groups, B*groups + B): the final step of sequence blockIdx.x -
// B*groups.  A grid's blocks are dispatched in index order, so when a final
// block starts every chunk block is running or done; it waits (bounded) for
// its sequence's records, and the finals of early sequences run while the
// last chunk blocks drain.
template <int DT>
__global__ __launch_bounds__(kBlock) void
#if SV_CHUNK_WAVES
__attribute__((amdgpu_waves_per_eu(SV_CHUNK_WAVES)))
#endif
k_chunks(const VerifyParams P)
{
    __shared__ double s_etab[kExpTabN];
    __shared__ __align__(16) double s_pool[kFinalPool];
    const int nblocks = P.B * P.groups;
    if ((int)blockIdx.x >= nblocks) {
        const int b = (int)blockIdx.x - nblocks;
        const SeqState s = P.seqs[b];
        // first read after sample_final's first barrier
        fill_exp_table(s_etab);
        sample_final<DT, false, false>(P, b, s, nullptr, s_etab, reinterpret_cast<ChunkSums*>(s_pool),
                                s_pool + kFinalPoolDoubles, nullptr);
        return;
    }
    const int b = (int)blockIdx.x / P.groups;
    const int g = (int)blockIdx.x - b * P.groups;
    const SeqState s = P.seqs[b];  // in flight with the table fill
    fill_exp_table(s_etab);
    __syncthreads();
    const int c0 = g * P.cpb, c1 = min(P.nch, c0 + P.cpb);
    const char* qrow = sample_qrow<DT>(P, b, s);
    const char* prow = s.mode == kModeResidual ? sample_prow<DT>(P, b, s) : qrow;
    const ExpRow eq = exp_row(P, s.mq, s_etab, nullptr), ep = exp_row(P, s.mp, s_etab, nullptr);
    const int cpw = (c1 - c0 + kWaves - 1) / kWaves;
    const int wave = (int)threadIdx.x >> 6;
    const int ca = min(c1, c0 + wave * cpw), cb = min(c1, ca + cpw);
    wave_chunks<DT>(P, b, s, qrow, prow, ca, cb, eq, ep, s_etab);
}

// ---------------------------------------------------------------------------
// Chain sample step of bf16 logits in 16-byte aligned rows: the table path
// ---------------------------------------------------------------------------
// Whether sequence b's chunks take the table: both rows it samples from do.
__device__ __forceinline__ bool tab_rows(const SeqState& s, const ExpRow& eq, const ExpRow& ep)
{
    return s.status == 0 && eq.tabbed && (s.mode != kModeResidual || ep.tabbed);
}

// The wave of a sequence's chunk blocks that forms the partial last chunk:
// the first wave without whole chunks in the sequence's last block (every
// block layout used leaves one there), else wave 0 of the first block.  So
// no wave carries both a whole chunk and the partial one.
__device__ __forceinline__ bool partial_wave(int whole, int cpb, int groups, int g, int wave)
{
    const int l0 = (groups - 1) * cpb, l1 = min(whole, l0 + cpb);
    int used = 0;
    if (l1 > l0) {
        const int lcpw = (l1 - l0 + kWaves - 1) / kWaves;
        used = (l1 - l0 + lcpw - 1) / lcpw;
    }
    return used < kWaves ? (g == groups - 1 && wave == used) : (g == 0 && wave == 0);
}

template <bool ONE>
__device__ __forceinline__ void tab_block_chunks(const VerifyParams& P, int b, int g, int cpb, int groups,
                                                 const SeqState& s, bool copied, double* s_etab, double* s_buf);

// Chunk block (b, g) of a chain: the sums of group g of the chunks of the
// row(s) sequence b samples from.  bf16 logits in 16-byte aligned rows
// (tab_block_chunks): each exponential one read of the block's LDS copy of
// the table, one contiguous share of the whole chunks per wave, each wave's
// first loads in flight while the table is copied; one wave (partial_wave)
// forms the partial last chunk; a sequence whose rows do not take the table
// (a row maximum beyond kTabRefLimit in units of T) has its chunks formed
// through exp_rel instead.  fp32 logits: every chunk through exp_rel.  ONE:
// the accept state and the table come from the same launch (polled; the
// table read through coherent loads).
template <int DT, bool ONE>
__device__ __forceinline__ void chunk_block_tab(const VerifyParams& P, int b, int g, int cpb, int groups,
                                                double* s_etab, double* s_buf)
{
    fill_exp_table(s_etab);
    if constexpr (DT != DT_BF16) {
        // rows without the table (fp32 logits): b's state, then this
        // group's chunks through exp_rel, the last group's up to nch
        const SeqState st = ONE ? wait_seq_state(P, b) : P.seqs[b];
        if (st.status) return;  // the final step emits the failure
        __syncthreads();        // s_etab
        const int wave = (int)threadIdx.x >> 6;
        const int c0 = g * cpb, c1 = (g == groups - 1) ? P.nch : min(P.nch, c0 + cpb);
        const int cpw = (c1 - c0 + kWaves - 1) / kWaves;
        const int ca = min(c1, c0 + wave * cpw), cb = min(c1, ca + cpw);
        const char* qrow = sample_qrow<DT>(P, b, st);
        const char* prow = st.mode == kModeResidual ? sample_prow<DT>(P, b, st) : qrow;
        const ExpRow rq = exp_row(P, st.mq, s_etab, nullptr), rp = exp_row(P, st.mp, s_etab, nullptr);
        wave_chunks<DT>(P, b, st, qrow, prow, ca, cb, rq, rp, s_etab);
        return;
    }
    SeqState s;
    bool copied = false;
    if constexpr (ONE) {
        // if b's accept state is not there yet, the table is copied while
        // waiting for it; if it is, the first row loads go out first
        u32x4 a[4];
        const bool mine =
            try_record<4>(make_rsrc(P.seqs, (size_t)P.B * kSeqStateBytes), (uint32_t)b * kSeqStateBytes, a, P.epoch);
        if (!__syncthreads_and(mine)) {
            if (!wait_value_table(P)) return;  // never expected: the final step times out and fails b
            copy_value_table_coherent(P, s_buf);
            copied = true;
        }
        s = wait_seq_state(P, b);
    } else {
        s = P.seqs[b];
    }
    tab_block_chunks<ONE>(P, b, g, cpb, groups, s, copied, s_etab, s_buf);
}

// The chunk work of block (b, g) given b's state (the table path; see
// chunk_block_tab).  copied: the table is in s_buf already.  With !ONE the
// table was filled by an earlier launch and is read with plain loads.
// s_etab holds the exp_rel table (fill_exp_table, published by a barrier
// here before any use).
template <bool ONE>
__device__ __forceinline__ void tab_block_chunks(const VerifyParams& P, int b, int g, int cpb, int groups,
                                                 const SeqState& s, bool copied, double* s_etab, double* s_buf)
{
    const ExpRow eq = exp_row(P, s.mq, s_etab, s_buf), ep = exp_row(P, s.mp, s_etab, s_buf);
    const int wave = (int)threadIdx.x >> 6;
    const char* qrow = sample_qrow<DT_BF16>(P, b, s);
    const char* prow = s.mode == kModeResidual ? sample_prow<DT_BF16>(P, b, s) : qrow;
    if (!tab_rows(s, eq, ep)) {
        if (s.status) return;  // the final step emits the failure
        // through exp_rel: this group's chunks, the last group's up to nch
        __syncthreads();
        const int c0 = g * cpb, c1 = (g == groups - 1) ? P.nch : min(P.nch, c0 + cpb);
        const int cpw = (c1 - c0 + kWaves - 1) / kWaves;
        const int ca = min(c1, c0 + wave * cpw), cb = min(c1, ca + cpw);
        const ExpRow rq = exp_row(P, s.mq, s_etab, nullptr), rp = exp_row(P, s.mp, s_etab, nullptr);
        wave_chunks<DT_BF16>(P, b, s, qrow, prow, ca, cb, rq, rp, s_etab);
        return;
    }
    const int whole = P.V / kChunk;
    const int c0 = g * cpb, c1 = min(whole, c0 + cpb);
    const int cpw = (c1 - c0 + kWaves - 1) / kWaves;
    const int ca = min(c1, c0 + wave * cpw), cb = min(c1, ca + cpw);
    const bool residual = s.mode == kModeResidual;
    const bool partial = P.nch > whole && partial_wave(whole, cpb, groups, g, wave);
    TabSlots sl;
    if (residual) tab_first_loads<false>(qrow, prow, ca, cb, sl);
    else tab_first_loads<true>(qrow, prow, ca, cb, sl);
    if constexpr (ONE) {
        if (!copied) {
            if (!wait_value_table(P)) return;  // never expected: the final step times out and fails b
            copy_value_table_coherent(P, s_buf);
        }
    } else {
        copy_value_table(P, s_buf);
    }
    __syncthreads();
    if (residual) {
        if (partial) partial_chunk_tab<false>(P, b, s, qrow, prow, whole, eq, ep, (lds_cptr)s_buf);
        chunk_range_tab<false>(P, b, s, qrow, prow, ca, cb, eq, ep, (lds_cptr)s_buf, sl);
    } else {
        if (partial) partial_chunk_tab<true>(P, b, s, qrow, prow, whole, eq, ep, (lds_cptr)s_buf);
        chunk_range_tab<true>(P, b, s, qrow, prow, ca, cb, eq, ep, (lds_cptr)s_buf, sl);
    }
}

// Final-step block of sequence b (exp_rel for the rescan; the chunk records
// are polled).
template <int DT, bool ONE>
__device__ __forceinline__ void final_block_tab(const VerifyParams& P, int b, double* s_etab, double* s_buf)
{
    const SeqState s = ONE ? wait_seq_state(P, b) : P.seqs[b];
    fill_exp_table(s_etab);  // first read after sample_final's first barrier
    sample_final<DT, false, false>(P, b, s, nullptr, s_etab, reinterpret_cast<ChunkSums*>(s_buf),
                                   s_buf + kFinalPoolDoubles, nullptr);
}

// LDS of the table path's blocks: the table (chunk blocks), the final step's
// records and band sums, or the accept test's row statistics.
constexpr int kTabBuf = kTabEntries > kFinalPool ? kTabEntries : kFinalPool;
static_assert((2 * kMaxChainN + 1) * sizeof(RowStat) <= kFinalPool * sizeof(double), "accept rows fit the buffer");

// The sample step of chains of bf16 logits in 16-byte aligned rows, after
// the row launch (which filled the table and ran the accept tests).  Blocks
// [0, B*groups): chunk block (b, g) is block g*B + b (groups of one
// sequence far apart in the grid stream faster than neighbouring ones).
// Blocks [B*groups, B*groups + B): the final step of one sequence each.
// Blocks are dispatched in index order: a final block waits (bounded) only
// on chunk blocks that have started.
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_sample_tab(const VerifyParams P)
{
    __shared__ double s_etab[kExpTabN];
    __shared__ __align__(16) double s_buf[kTabBuf];
    const int nblocks = P.B * P.groups;
    if ((int)blockIdx.x >= nblocks) {
        final_block_tab<DT_BF16, false>(P, (int)blockIdx.x - nblocks, s_etab, s_buf);
        return;
    }
    const int g = (int)blockIdx.x / P.B;
    chunk_block_tab<DT_BF16, false>(P, (int)blockIdx.x - g * P.B, g, P.cpb, P.groups, s_etab, s_buf);
}

// The whole chain step in one launch: bf16 logits in 16-byte aligned rows
// (with the table) and fp32 logits (chunk sums through exp_rel, no table).
// Blocks [0, tab_blocks) fill the table; the rest form sections (see
// VerifyParams::sched): section k holds the row blocks of sequence group k,
// then the accept blocks of group k - fuse_la, the chunk blocks of group
// k - fuse_lc (group-major within the group) and the final blocks of group
// k - fuse_lf.  Every block waits only on blocks before it (rows <- accept
// <- chunks <- finals, table <- chunks), which the in-order dispatch has
// started, and every wait is bounded.  Sample work of early groups thus runs
// while later groups' rows still stream.
template <int DT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_chain_tab(const VerifyParams P)
{
    __shared__ double s_etab[kExpTabN];
    // bf16: the table (chunk blocks) or the final step's records; fp32 rows
    // have no table
    __shared__ __align__(16) double s_buf[DT == DT_BF16 ? kTabBuf : kFinalPool];
    int x = (int)blockIdx.x;
    if (x < P.tab_blocks) {
        fill_value_table(P, x);
        return;
    }
    x -= P.tab_blocks;
    int lo = 0, hi = P.fuse_nsec;  // the section: the last k with sched[k] <= x
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (P.sched[mid] <= x) lo = mid;
        else hi = mid;
    }
    const int k = lo, ng = P.fuse_ng;
    int off = x - P.sched[k];
    if (k < ng) {
        const int n = (P.fuse_gstart[k + 1] - P.fuse_gstart[k]) * P.r_items;
        if (off < n) {
            const int r = off / P.r_items;
            row_block<DT, false>(P, P.fuse_gstart[k] + r, off - r * P.r_items);
            return;
        }
        off -= n;
    }
    int j = k - P.fuse_la;
    if (j >= 0 && j < ng) {
        const int n = P.fuse_gstart[j + 1] - P.fuse_gstart[j];
        if (off < n) {
            if (threadIdx.x < 64)
                chain_accept<DT>(P, P.fuse_gstart[j] + off, reinterpret_cast<RowStat*>(s_buf), true);
            return;
        }
        off -= n;
    }
    j = k - P.fuse_lc;
    if (j >= 0 && j < ng) {
        const int nj = P.fuse_gstart[j + 1] - P.fuse_gstart[j], n = nj * P.fuse_groups[j];
        if (off < n) {
            const int g = off / nj;
            chunk_block_tab<DT, true>(P, P.fuse_gstart[j] + off - g * nj, g, P.fuse_cpb[j], P.fuse_groups[j], s_etab,
                                      s_buf);
            return;
        }
        off -= n;
    }
    j = k - P.fuse_lf;  // the rest of the section: final blocks
    if (j < 0 || j >= ng || off >= P.fuse_gstart[j + 1] - P.fuse_gstart[j]) return;  // not reached: sched is exact
    final_block_tab<DT, true>(P, P.fuse_gstart[j] + off, s_etab, s_buf);
}

// Sample kernel: block (b, group) reads b's accept state and walk path (from
// the accept blocks of the row launch), forms the chunk sums of its group of
// chunks of the row(s) b samples from, and the last of b's blocks to finish
// (an arrival counter per sequence) runs b's final step.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_sample(const VerifyParams P)
{
    const int b = (int)blockIdx.x / P.groups;
    const int g = (int)blockIdx.x - b * P.groups;
    __shared__ SeqState s_state;
    __shared__ int32_t s_path[kMaxNodes];
    __shared__ double s_etab[kExpTabN];
    // bf16: the table for the chunk sums, then the final step's records
    __shared__ __align__(16) double s_pool[DT == DT_BF16 ? kTabBuf : kFinalPool];
    fill_exp_table(s_etab);
    if (threadIdx.x == 0) s_state = P.seqs[b];
    const int plen = min(P.nn, P.max_depth + 1);
    for (int i = (int)threadIdx.x; i < plen; i += kBlock) s_path[i] = P.paths[(int64_t)b * P.nn + i];
    __syncthreads();
    const SeqState s = s_state;
    bool tab = false;
    if constexpr (DT == DT_BF16) {
        if (P.use_tab) {
            // bf16 rows with the call's table (filled by the row launch)
            tab_block_chunks<false>(P, b, g, P.cpb, P.groups, s, false, s_etab, s_pool);
            tab = true;
        }
    }
    if (!tab) {
        const int c0 = g * P.cpb, c1 = min(P.nch, c0 + P.cpb);
        const char* qrow = sample_qrow<DT>(P, b, s);
        const char* prow = s.mode == kModeResidual ? sample_prow<DT>(P, b, s) : qrow;
        const ExpRow eq = exp_row(P, s.mq, s_etab, nullptr), ep = exp_row(P, s.mp, s_etab, nullptr);
        // each wave takes a contiguous share of the block's chunks; whole
        // chunks of aligned rows stream with loads in flight across chunk
        // boundaries
        const int cpw = (c1 - c0 + kWaves - 1) / kWaves;
        const int wave = (int)threadIdx.x >> 6;
        const int ca = min(c1, c0 + wave * cpw), cb = min(c1, ca + cpw);
        wave_chunks<DT>(P, b, s, qrow, prow, ca, cb, eq, ep, s_etab);
    }
    __syncthreads();
    __shared__ int s_last;
    if (threadIdx.x == 0) s_last = arrive(P.chunk_arrivals + b, P.epoch) == (uint32_t)(P.groups - 1);
    __syncthreads();
    if (s_last)
        sample_final<DT, true, false>(P, b, s, s_path, s_etab, reinterpret_cast<ChunkSums*>(s_pool),
                                      s_pool + kFinalPoolDoubles, nullptr);
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

// Row segments of about SV_SEG_TARGET elements (a multiple of 64 elements,
// so every segment keeps the row's 16-byte alignment): one row block each.
#ifndef SV_SEG_TARGET
#define SV_SEG_TARGET 65536
#endif
constexpr int kSegTarget = SV_SEG_TARGET;
void segments_of(int V, int* segs, int* seg_len)
{
    int s = (V + kSegTarget - 1) / kSegTarget;
    if (s < 1) s = 1;
    int len = (V + s - 1) / s;
    len = (len + 63) / 64 * 64;
    *seg_len = len;
    *segs = (V + len - 1) / len;
}


// Blocks of a kernel the device holds at once (compute units x occupancy).
template <typename K>
int resident_blocks(K kernel, std::atomic<int>& cache, int block = sv::kBlock)
{
    int v = cache.load();
    if (v) return v;
    int dev = 0, cus = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kernel), block, 0) !=
            hipSuccess ||
        occ <= 0)
        return 0;
    v = cus * occ;
    cache.store(v);
    return v;
}

struct Layout {
    size_t chunk_arr, seqs, paths, stats, part, tab, tab_done, total;
};

// path_len: int32 entries per sequence of the walk's path (trees: nodes)
Layout make_layout(int B, int rows, int V, int path_len = 0)
{
    int segs, seg_len;
    segments_of(V, &segs, &seg_len);
    Layout L;
    L.chunk_arr = 0;
    L.seqs = L.chunk_arr + align_up((size_t)B * sizeof(uint64_t));
    L.paths = L.seqs + align_up((size_t)B * sizeof(sv::SeqState));
    L.stats = L.paths + align_up((size_t)B * path_len * sizeof(int32_t));
    L.part = L.stats + align_up((size_t)B * rows * segs * sv::kRowStatBytes);
    L.tab = L.part + align_up((size_t)B * nchunks_of(V) * sv::kChunkSumsBytes);
    L.tab_done = L.tab + align_up((size_t)sv::kTabEntries * sizeof(double));
    L.total = L.tab_done + align_up((size_t)((sv::kTabEntries + sv::kBlock - 1) / sv::kBlock) * 16);
    return L;
}

// The record regions are addressed with 32-bit buffer offsets.
bool regions_fit(const Layout& L)
{
    return L.part - L.stats <= (size_t)INT32_MAX && L.tab - L.part <= (size_t)INT32_MAX;
}

// The bf16-grid table of a temperature: binades [2^(e-12), 2^(e+7)), e =
// floor(log2 T), as magnitude keys from `lo`; false where that range leaves
// the normal bf16 exponents (then calls use exp_rel throughout).
#ifndef SV_VALUE_TABLE
#define SV_VALUE_TABLE 1
#endif
bool value_table_range(float T, uint32_t* lo)
{
    int e2 = 0;
    frexp((double)T, &e2);  // T = f 2^e2, f in [0.5, 1)
    const int blo = 127 + (e2 - 1) - 12;
    if (!SV_VALUE_TABLE || blo < 1 || blo + sv::kTabBinades > 255) return false;
    *lo = (uint32_t)blo << 7;
    return true;
}

// Logit rows of B sequences x nrows rows x V elements of es bytes.
int check_rows(const void* base, int64_t seq_stride, int64_t row_stride, int es, int B, int nrows, int V)
{
    if (((uintptr_t)base % (uintptr_t)es) != 0) return SV_EALIGN;
    if (seq_stride < 0 || row_stride < 0) return SV_EINVAL;
    if (seq_stride > INT64_MAX / es || row_stride > INT64_MAX / es) return SV_EINVAL;
    if (!sv::span_fits(B, seq_stride * es, nrows, row_stride * es, 1, 0, (int64_t)V * es)) return SV_EINVAL;
    return SV_OK;
}

// Calls are numbered by a 64-bit counter that starts at a value drawn when
// the library is loaded (so a reloaded library does not repeat the numbers
// of the instance before it); records and counters carry the low word.
uint64_t epoch_start()
{
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    const uint64_t a = (uint64_t)(uintptr_t)&t;
    uint64_t x = t ^ (a << 17) ^ (uint64_t)std::random_device{}();
    x ^= x >> 33;
    x *= 0xff51afd7ed558ccdull;
    x ^= x >> 33;
    return x;
}
std::atomic<uint64_t> g_epoch{epoch_start()};
uint32_t next_epoch()
{
    uint32_t e;
    do {
        e = (uint32_t)(g_epoch.fetch_add(1) + 1);
    } while (e == 0);
    return e;
}

// The bound of the kernels' waits for records of other blocks: kSpinLimit
// polls, or the value of SV_TEST_SPIN_LIMIT in the environment (tests of the
// timeout path set it to a few polls; every wait stays bounded either way).
int spin_limit_for_call()
{
    const char* e = getenv("SV_TEST_SPIN_LIMIT");
    if (e && *e) {
        char* end = nullptr;
        const long v = strtol(e, &end, 10);
        if (end && *end == 0 && v >= 0 && v <= sv::kSpinLimit) return (int)v;
    }
    return sv::kSpinLimit;
}

// Sample blocks per sequence: enough for one round of the blocks the device
// holds at once (a block's four waves share its chunks).
template <int DT>
void set_groups(sv::VerifyParams& P)
{
    static std::atomic<int> cache{0};
    const int resident = resident_blocks(&sv::k_sample<DT>, cache);
    int groups = resident > 0 ? resident / (P.B > 0 ? P.B : 1) : 1;
    groups = groups < 1 ? 1 : (groups > P.nch ? P.nch : groups);
    P.cpb = (P.nch + groups - 1) / groups;
    P.groups = (P.nch + P.cpb - 1) / P.cpb;
}

// Chunk-sum blocks per sequence (chains): about SV_CHUNKS_PER_BLOCK chunks
// each, SV_TAB_CHUNKS_PER_BLOCK with the bf16-grid table (each block copies
// the table into LDS first, so fewer blocks carry more chunks).
#ifndef SV_CHUNKS_PER_BLOCK
#define SV_CHUNKS_PER_BLOCK 4
#endif
#ifndef SV_TAB_CHUNKS_PER_BLOCK
#define SV_TAB_CHUNKS_PER_BLOCK 8
#endif
// Whole chunks per tree sample block on the table path (each such block
// also copies the table into LDS).
#ifndef SV_TREE_CHUNKS_PER_BLOCK
#define SV_TREE_CHUNKS_PER_BLOCK SV_TAB_CHUNKS_PER_BLOCK
#endif
// The table path in one launch (k_chain_tab) rather than a row launch and a
// sample launch; sequences per section, and the lags (in sections) of a
// group's accept, chunk and final blocks behind its row blocks.
#ifndef SV_ONE_LAUNCH
#define SV_ONE_LAUNCH 1
#endif
#ifndef SV_FUSE_GROUP
#define SV_FUSE_GROUP 16
#endif
#ifndef SV_FUSE_TAIL_GROUPS
#define SV_FUSE_TAIL_GROUPS 0
#endif
#ifndef SV_FUSE_TAIL_GROUP
#define SV_FUSE_TAIL_GROUP 4
#endif
#ifndef SV_LAZY_BONUS
#define SV_LAZY_BONUS 1
#endif
#ifndef SV_TAIL_CHUNKS_PER_BLOCK
#define SV_TAIL_CHUNKS_PER_BLOCK 4
#endif
#ifndef SV_FUSE_LA
#define SV_FUSE_LA 2
#endif
#ifndef SV_FUSE_LC
#define SV_FUSE_LC 4
#endif
#ifndef SV_FUSE_LF
#define SV_FUSE_LF 6
#endif
// The row kernel; with a timing hook, its begin and rows_done events are
// stamped by the kernel's own start and end (not by records beside it, whose
// interval would also hold the dispatch gap before the kernel).
template <int DT, bool TREE>
void launch_rows(const sv::VerifyParams& P, int64_t grid, const sv_timing* timing, hipStream_t stream)
{
    const hipEvent_t t0 = timing ? timing->begin : nullptr;
    const hipEvent_t t1 = timing ? timing->rows_done : nullptr;
    hipExtLaunchKernelGGL((sv::k_rows<DT, TREE>), dim3((unsigned)grid), dim3(sv::kBlock), 0, stream, t0, t1, 0, P);
}

// Chains: the row kernel (row statistics, table, accept tests), then the
// sample step: with the bf16-grid table, the table's chunk kernel and the
// final kernel; otherwise one kernel of chunk sums and finals.
template <int DT>
int launch_chain(sv::VerifyParams& P, const sv_timing* timing, hipStream_t stream)
{
    const hipEvent_t t_end = timing ? timing->end : nullptr;
#if SV_ONE_LAUNCH
    // one launch: bf16 rows with the table, and fp32 rows (whose chunk
    // blocks go through exp_rel); bf16 rows that are not 16-byte aligned
    // take the two launches below
    const bool one = P.use_tab || DT == sv::DT_F32;
#else
    const bool one = false;
#endif
    if (one) {
        // the bonus row is read only by the sequences that sample from it
        P.lazy_bonus = SV_LAZY_BONUS;
        if (P.lazy_bonus) P.r_items = (P.rows - 1) * P.segs;
        // sections of sequence groups (at most 64): groups of SV_FUSE_GROUP,
        // then SV_FUSE_TAIL_GROUPS of SV_FUSE_TAIL_GROUP (smaller last groups
        // leave less sample work for the end; measured slower at B=256, so
        // none by default)
        int tg = SV_FUSE_TAIL_GROUPS, tgs = SV_FUSE_TAIL_GROUP;
        if ((int64_t)tg * tgs * 2 > P.B) tg = 0;
        const int main_b = P.B - tg * tgs;
        int gs = SV_FUSE_GROUP;
        gs = gs < (main_b + 63 - tg) / (64 - tg) ? (main_b + 63 - tg) / (64 - tg) : gs;
        gs = gs < 1 ? 1 : gs;
        int ng = 0;
        for (int b0 = 0; b0 < main_b; b0 += gs) P.fuse_gstart[ng++] = b0;
        for (int t = 0; t < tg; ++t) P.fuse_gstart[ng++] = main_b + t * tgs;
        P.fuse_gstart[ng] = P.B;
        P.fuse_ng = ng;
        P.fuse_la = SV_FUSE_LA < ng ? SV_FUSE_LA : ng;
        P.fuse_lc = SV_FUSE_LC < ng ? SV_FUSE_LC : ng;
        P.fuse_lf = SV_FUSE_LF < ng ? SV_FUSE_LF : ng;
        P.fuse_lc = P.fuse_lc < P.fuse_la ? P.fuse_la : P.fuse_lc;
        P.fuse_lf = P.fuse_lf < P.fuse_lc ? P.fuse_lc : P.fuse_lf;
        P.fuse_nsec = ng + P.fuse_lf;
        // chunk blocks per sequence: the table path splits the whole chunks
        // (the partial one goes to an idle wave), exp_rel splits every chunk
        const int span = P.use_tab ? P.V / sv::kChunk : P.nch;
        for (int j = 0; j < ng; ++j) {
            const int want = !P.use_tab ? SV_CHUNKS_PER_BLOCK
                             : j + P.fuse_lc >= ng ? SV_TAIL_CHUNKS_PER_BLOCK : SV_TAB_CHUNKS_PER_BLOCK;
            int gj = (span + want - 1) / want;
            gj = gj < 1 ? 1 : gj;
            int cj = (span + gj - 1) / gj;
            cj = cj < 1 ? 1 : cj;
            P.fuse_cpb[j] = (int16_t)cj;
            P.fuse_groups[j] = (int16_t)gj;
        }
        auto nseq = [&](int j) -> int64_t { return (j >= 0 && j < ng) ? P.fuse_gstart[j + 1] - P.fuse_gstart[j] : 0; };
        auto nchunkb = [&](int j) -> int64_t { return (j >= 0 && j < ng) ? nseq(j) * P.fuse_groups[j] : 0; };
        int64_t at = 0;
        for (int k = 0; k < P.fuse_nsec; ++k) {
            P.sched[k] = (int)at;
            at += nseq(k) * P.r_items + nseq(k - P.fuse_la) + nchunkb(k - P.fuse_lc) + nseq(k - P.fuse_lf);
        }
        P.sched[P.fuse_nsec] = (int)at;
        const hipEvent_t t0 = timing ? timing->begin : nullptr;
        const hipEvent_t t1 = timing ? timing->rows_done : nullptr;
        hipExtLaunchKernelGGL((sv::k_chain_tab<DT>), dim3((unsigned)(P.tab_blocks + at)), dim3(sv::kBlock), 0,
                              stream, t0, t1, 0, P);
        if (t_end && hipEventRecord(t_end, stream) != hipSuccess) return SV_EHIP;
    } else if (P.use_tab) {
        const int whole = P.V / sv::kChunk;
        int groups = (whole + SV_TAB_CHUNKS_PER_BLOCK - 1) / SV_TAB_CHUNKS_PER_BLOCK;
        groups = groups < 1 ? 1 : groups;
        P.cpb = (whole + groups - 1) / groups;
        P.cpb = P.cpb < 1 ? 1 : P.cpb;
        P.groups = groups;
        launch_rows<DT, false>(P, (int64_t)P.B * (P.r_items + 1) + P.tab_blocks, timing, stream);
        // chunk-sum blocks, then one final-step block per sequence
        hipExtLaunchKernelGGL(sv::k_sample_tab, dim3((unsigned)((int64_t)P.B * (P.groups + 1))), dim3(sv::kBlock), 0,
                              stream, nullptr, t_end, 0, P);
    } else {
        int groups = (P.nch + SV_CHUNKS_PER_BLOCK - 1) / SV_CHUNKS_PER_BLOCK;
        groups = groups < 1 ? 1 : groups;
        P.cpb = (P.nch + groups - 1) / groups;
        P.groups = (P.nch + P.cpb - 1) / P.cpb;
        launch_rows<DT, false>(P, (int64_t)P.B * (P.r_items + 1) + P.tab_blocks, timing, stream);
        // chunk-sum blocks, then one final-step block per sequence
        hipExtLaunchKernelGGL((sv::k_chunks<DT>), dim3((unsigned)((int64_t)P.B * (P.groups + 1))),
                              dim3(sv::kBlock), 0, stream, nullptr, t_end, 0, P);
    }
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    return SV_OK;
}

// Trees: the row kernel, then the sample kernel.
template <int DT>
int launch_tree(sv::VerifyParams& P, const sv_timing* timing, hipStream_t stream)
{
    if (P.use_tab) {
        // table path: blocks of about SV_TREE_CHUNKS_PER_BLOCK whole chunks
        // (each block copies the table), but no
        // more than one round of the blocks the device holds at once
        static std::atomic<int> cache{0};
        const int resident = resident_blocks(&sv::k_sample<DT>, cache);
        const int whole = P.V / sv::kChunk;
        int groups = (whole + SV_TREE_CHUNKS_PER_BLOCK - 1) / SV_TREE_CHUNKS_PER_BLOCK;
        const int round = resident > 0 && P.B > 0 ? resident / P.B : groups;
        groups = groups > round ? round : groups;
        groups = groups < 1 ? 1 : groups;
        P.cpb = (whole + groups - 1) / groups;
        P.cpb = P.cpb < 1 ? 1 : P.cpb;
        P.groups = groups;
    } else {
        set_groups<DT>(P);
    }
    const int64_t row_grid = (int64_t)P.B * P.r_items + P.tab_blocks + P.B;
    const int64_t sample_grid = (int64_t)P.B * P.groups;
    launch_rows<DT, true>(P, row_grid, timing, stream);
    hipExtLaunchKernelGGL((sv::k_sample<DT>), dim3((unsigned)sample_grid), dim3(sv::kBlock), 0, stream, nullptr,
                          timing ? timing->end : nullptr, 0, P);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    return SV_OK;
}

template <bool TREE>
int launch_verify(sv::VerifyParams& P, int dtype, void* workspace, const Layout& L, const sv_timing* timing,
                  hipStream_t stream)
{
    char* ws = static_cast<char*>(workspace);
    P.chunk_arrivals = reinterpret_cast<uint64_t*>(ws + L.chunk_arr);
    P.seqs = reinterpret_cast<sv::SeqState*>(ws + L.seqs);
    P.paths = reinterpret_cast<int32_t*>(ws + L.paths);
    P.stats = ws + L.stats;
    P.part = ws + L.part;
    P.etab_g = reinterpret_cast<double*>(ws + L.tab);
    P.tab_done = ws + L.tab_done;
    P.stats_bytes = (uint32_t)(L.part - L.stats);
    P.part_bytes = (uint32_t)(L.tab - L.part);
    // the table path: chains of bf16 logits whose rows are all 16-byte aligned
    const bool aligned = (((uintptr_t)P.zq | (uintptr_t)P.zp) & 15u) == 0 && P.qs % 8 == 0 && P.qr % 8 == 0 &&
                         P.ps % 8 == 0 && P.pr % 8 == 0;
    P.use_tab = dtype == SV_BF16 && aligned && value_table_range(P.T, &P.tab_lo) ? 1 : 0;
    P.tab_blocks = P.use_tab ? (sv::kTabEntries + sv::kBlock - 1) / sv::kBlock : 0;
    P.epoch = next_epoch();
    P.spin_limit = spin_limit_for_call();
    if constexpr (!TREE)
        return dtype == SV_BF16 ? launch_chain<sv::DT_BF16>(P, timing, stream)
                                : launch_chain<sv::DT_F32>(P, timing, stream);
    else
        return dtype == SV_BF16 ? launch_tree<sv::DT_BF16>(P, timing, stream)
                                : launch_tree<sv::DT_F32>(P, timing, stream);
}

void fill_common(sv::VerifyParams& P, int B, int V, int rows, uint64_t seed, uint64_t round, float temperature)
{
    P.B = B;
    P.V = V;
    P.rows = rows;
    segments_of(V, &P.segs, &P.seg_len);
    P.r_items = rows * P.segs;
    P.nch = nchunks_of(V);
    P.seed = seed;
    P.round = round;
    P.T = temperature;
    P.invT = 1.0 / (double)temperature;
    P.cd = 1.4426950408889634074 / (double)temperature;  // log2(e) / T
    P.c = (float)P.cd;
}

// Grids must fit an unsigned launch dimension.
bool item_count_ok(int B, int rows, int V)
{
    int segs, seg_len;
    segments_of(V, &segs, &seg_len);
    return 2 * (int64_t)B * rows * segs + 64 < (int64_t)INT32_MAX && (int64_t)B * (nchunks_of(V) + 1) < (int64_t)INT32_MAX;
}

}  // namespace

// Workspace of spec_verify_chain_noalloc: device memory of the library
// itself, zero when the library is loaded, one copy per GPU.  In host code
// the name only stands for the symbol; the device address comes from
// hipGetSymbolAddress (scratch_on_current_device).
static __device__ __align__(256) char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_on_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SV_OK;
}

}  // namespace

extern "C" {

int sv_abi_version(void) { return 6; }

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
        case SV_ESCRATCH: return "sizes exceed the no-allocation entry point's static scratch";
        default: return "unknown status";
    }
}

size_t sv_chain_workspace_bytes(int B, int N, int V)
{
    if (B < 0 || N < 0 || N > 64 || V < 1 || V > sv::kMaxChunks * sv::kChunk) return 0;
    return make_layout(B, 2 * N + 1, V).total;
}

size_t sv_tree_workspace_bytes(int B, int T, int V)
{
    if (B < 0 || T < 0 || T >= sv::kMaxNodes || V < 1 || V > sv::kMaxChunks * sv::kChunk) return 0;
    return make_layout(B, 2 * (T + 1), V, T + 1).total;
}

int spec_verify_chain(const void* target_logits, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                      const void* draft_logits, int64_t drf_seq_stride, int64_t drf_row_stride, int dtype,
                      const int32_t* draft_tokens, int B, int N, int V, uint64_t seed, uint64_t round,
                      float temperature, int32_t* out_tokens, int32_t* out_num_accepted, int8_t* out_accept,
                      float* out_probs, double* out_residual_mass, const int32_t* kv_len_in, int32_t* out_src_rows,
                      int32_t* out_kv_len, void* workspace, size_t workspace_bytes, const sv_timing* timing,
                      hipStream_t stream)
{
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
    if (B < 0 || N < 0 || V < 1 || !(temperature > 0.0f) || !(temperature < INFINITY)) return SV_EINVAL;
    if (N > 64 || V > sv::kMaxChunks * sv::kChunk) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!target_logits || !out_tokens || !out_num_accepted) return SV_EINVAL;
    if (N > 0 && (!draft_logits || !draft_tokens)) return SV_EINVAL;
    if ((out_src_rows || out_kv_len) && !kv_len_in) return SV_EINVAL;
    const int es = dtype == SV_BF16 ? 2 : 4;
    int rc = check_rows(target_logits, tgt_seq_stride, tgt_row_stride, es, B, N + 1, V);
    if (rc) return rc;
    if (N > 0 && (rc = check_rows(draft_logits, drf_seq_stride, drf_row_stride, es, B, N, V))) return rc;
    if (!item_count_ok(B, 2 * N + 1, V)) return SV_ESHAPE;
    const Layout L = make_layout(B, 2 * N + 1, V);
    if (!regions_fit(L)) return SV_ESHAPE;
    if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 15u)) return SV_EWORKSPACE;

    sv::VerifyParams P{};
    P.zq = static_cast<const char*>(target_logits);
    P.zp = static_cast<const char*>(draft_logits ? draft_logits : target_logits);
    P.qs = tgt_seq_stride;
    P.qr = tgt_row_stride;
    P.ps = drf_seq_stride;
    P.pr = drf_row_stride;
    P.tokens = draft_tokens;
    P.parents = nullptr;
    P.parents_shared = 1;
    P.N = N;
    P.nn = N + 1;
    P.max_depth = N;
    P.width = N + 1;
    fill_common(P, B, V, 2 * N + 1, seed, round, temperature);
    P.out_tokens = out_tokens;
    P.out_path = nullptr;
    P.out_num = out_num_accepted;
    P.out_acc = out_accept;
    P.out_probs = out_probs;
    P.out_resid = out_residual_mass;
    P.kv_len_in = kv_len_in;
    P.out_src_rows = out_src_rows;
    P.out_kv_len = out_kv_len;
    return launch_verify<false>(P, dtype, workspace, L, timing, stream);
}

int spec_verify_chain_noalloc(const void* target_logits, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                              const void* draft_logits, int64_t drf_seq_stride, int64_t drf_row_stride, int dtype,
                              const int32_t* draft_tokens, int B, int N, int V, uint64_t seed, uint64_t round,
                              float temperature, int32_t* out_tokens, int32_t* out_num_accepted,
                              int8_t* out_accept, float* out_probs, double* out_residual_mass,
                              const int32_t* kv_len_in, int32_t* out_src_rows, int32_t* out_kv_len,
                              const sv_timing* timing, hipStream_t stream)
{
    // sizes the static scratch cannot hold are refused before any HIP call
    const size_t need = sv_chain_workspace_bytes(B, N, V);
    if (need > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ESCRATCH;
    if (B == 0 || need == 0)  // empty batch or invalid sizes: the regular entry point's status
        return spec_verify_chain(target_logits, tgt_seq_stride, tgt_row_stride, draft_logits, drf_seq_stride,
                                 drf_row_stride, dtype, draft_tokens, B, N, V, seed, round, temperature, out_tokens,
                                 out_num_accepted, out_accept, out_probs, out_residual_mass, kv_len_in, out_src_rows,
                                 out_kv_len, nullptr, 0, timing, stream);
    void* ws = nullptr;
    const int rc = scratch_on_current_device(&ws);
    if (rc) return rc;
    return spec_verify_chain(target_logits, tgt_seq_stride, tgt_row_stride, draft_logits, drf_seq_stride,
                             drf_row_stride, dtype, draft_tokens, B, N, V, seed, round, temperature, out_tokens,
                             out_num_accepted, out_accept, out_probs, out_residual_mass, kv_len_in, out_src_rows,
                             out_kv_len, ws, (size_t)SV_NOALLOC_SCRATCH_BYTES, timing, stream);
}

int spec_verify_tree(const void* target_logits, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                     const void* draft_logits, int64_t drf_seq_stride, int64_t drf_row_stride, int dtype,
                     const int32_t* node_tokens, const int32_t* parents, int parents_shared, int B, int T, int V,
                     int max_depth, int walk, uint64_t seed, uint64_t round, float temperature,
                     int32_t* out_tokens, int32_t* out_path_nodes, int32_t* out_num_accepted, int8_t* out_accept,
                     float* out_probs, double* out_residual_mass, const int32_t* kv_len_in, int32_t* out_src_rows,
                     int32_t* out_kv_len, void* workspace, size_t workspace_bytes, const sv_timing* timing,
                     hipStream_t stream)
{
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
    if (B < 0 || T < 0 || V < 1 || max_depth < 0 || !(temperature > 0.0f) || !(temperature < INFINITY) ||
        (walk != SV_WALK_FIRST_ACCEPTED && walk != SV_WALK_BEST_CHILD))
        return SV_EINVAL;
    if (T >= sv::kMaxNodes || max_depth > T || V > sv::kMaxChunks * sv::kChunk) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!target_logits || !draft_logits || !node_tokens || !parents || !out_tokens || !out_path_nodes ||
        !out_num_accepted)
        return SV_EINVAL;
    if ((out_src_rows || out_kv_len) && !kv_len_in) return SV_EINVAL;
    const int es = dtype == SV_BF16 ? 2 : 4;
    const int nn = T + 1;
    int rc = check_rows(target_logits, tgt_seq_stride, tgt_row_stride, es, B, nn, V);
    if (rc) return rc;
    if ((rc = check_rows(draft_logits, drf_seq_stride, drf_row_stride, es, B, nn, V))) return rc;
    if (!item_count_ok(B, 2 * nn, V)) return SV_ESHAPE;
    const Layout L = make_layout(B, 2 * nn, V, nn);
    if (!regions_fit(L)) return SV_ESHAPE;
    if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 15u)) return SV_EWORKSPACE;

    sv::VerifyParams P{};
    P.zq = static_cast<const char*>(target_logits);
    P.zp = static_cast<const char*>(draft_logits);
    P.qs = tgt_seq_stride;
    P.qr = tgt_row_stride;
    P.ps = drf_seq_stride;
    P.pr = drf_row_stride;
    P.tokens = node_tokens;
    P.parents = parents;
    P.parents_shared = parents_shared ? 1 : 0;
    P.N = 0;
    P.nn = nn;
    P.max_depth = max_depth;
    P.width = max_depth + 1;
    P.walk = walk;
    fill_common(P, B, V, 2 * nn, seed, round, temperature);
    P.out_tokens = out_tokens;
    P.out_path = out_path_nodes;
    P.out_num = out_num_accepted;
    P.out_acc = out_accept;
    P.out_probs = out_probs;
    P.out_resid = out_residual_mass;
    P.kv_len_in = kv_len_in;
    P.out_src_rows = out_src_rows;
    P.out_kv_len = out_kv_len;
    return launch_verify<true>(P, dtype, workspace, L, timing, stream);
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
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

}  // extern "C"
