/*
 * CPU ORACLE for the delta-prefetched sparse FFN -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load or call this file. The HIP library shares no code, header, table or
 * helper with it. It is deliberately plain and slow: scalar loops, no
 * blocking, no reordering beyond what the method states, fp64 arithmetic.
 *
 * What it computes (per sparse layer, per decode token), following
 * "NeuroPrefetcher: Storage-Aware Sparse LLM Inference via Delta
 * Prefetching" (Dhar et al.), section 3.4 "Predictive Delta Prefetching",
 * and its I/O path, section 3.5:
 *
 *   1. The predicted active set A_t is built from the gate-centroid and
 *      up-centroid bitmasks of the layer. The paper intersects them; the
 *      build's workloads use the union; a single-table mode serves a
 *      non-gated FFN. Bit b of word w is neuron 64*w + b.
 *   2. The resident buffer is updated by set difference:
 *        D_in  = A_t \ R_{t-1}   (incoming rows, fetched),
 *        D_out = R_{t-1} \ A_t   (outgoing rows, their slots released),
 *      both in ascending neuron order (incoming IDs are sorted before the
 *      reads are issued, section 3.5).
 *   3. Outgoing neurons release their slots: the slot map entry becomes -1
 *      and the slot is free. Freed rows keep their stale bytes.
 *   4. The i-th incoming neuron (ascending) takes the i-th free slot
 *      (ascending slot index), the slot map and the owner table are
 *      updated, and its [gate|up|down^T] bundle is copied into the slot.
 *      Persisting neurons keep their slot: no compaction.
 *   5. R_t = A_t. The first token (R empty) fetches the whole set.
 *   6. If |A_t| > K_max the step is refused and the state is unchanged.
 *
 * The FFN (section 3.4: row i of gate, up and down^T for each active
 * neuron i) is y = sum_{i in A_t} down_i * act(gate_i . x) * (up_i . x)
 * for the gated bundle, and y = sum_{i in A_t} down_i * act(up_i . x)
 * for the [up|down^T] bundle of a non-gated FFN (LLM in a flash, sections
 * 3.2 and 3.3). act is ReLU (the benchmark's gated-ReLU models) or SiLU,
 * silu(g) = g / (1 + exp(-g)), the gate of the SwiGLU MLPs the paper runs
 * (section 3.4). The oracle evaluates it straight from the row
 * store in fp64, over neuron IDs in the order given (callers pass them
 * ascending), without looking at the slot machinery. bf16 -> fp64 and
 * fp32 -> fp64 are exact, and so is each bf16 x fp32 product in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { NPO_UNION = 0, NPO_INTERSECT = 1, NPO_SINGLE = 2 };
enum { NPO_OK = 0, NPO_EINVAL = 1, NPO_ECAPACITY = 2 };

static int npo_bit(const uint64_t* words, int32_t n) {
    return (int)((words[n / 64] >> (n % 64)) & 1ULL);
}

/*
 * Step 1: active set. Writes the ascending neuron IDs to S (capacity M) and
 * returns their count, or -1 for an unknown mode. mask_u is ignored in
 * single mode.
 */
int32_t npo_active_set(const uint64_t* mask_g, const uint64_t* mask_u, int32_t M, int32_t mode,
                       int32_t* S) {
    int32_t n = 0;
    for (int32_t i = 0; i < M; ++i) {
        int g = npo_bit(mask_g, i);
        int member;
        if (mode == NPO_UNION) {
            member = g || npo_bit(mask_u, i);
        } else if (mode == NPO_INTERSECT) {
            member = g && npo_bit(mask_u, i);
        } else if (mode == NPO_SINGLE) {
            member = g;
        } else {
            return -1;
        }
        if (member) S[n++] = i;
    }
    return n;
}

/*
 * Steps 2-6 for one layer. State arrays belong to the caller:
 *   slot_map[M]: slot of neuron n, or -1 when n is not resident;
 *   owner[K]:    neuron held by slot s, or -1 when the slot is free.
 * S[n_active] is the new active set (ascending, distinct, < M).
 * Outputs (capacity K each): d_in / slot_in (n_in entries), d_out (n_out).
 * Returns NPO_ECAPACITY, state untouched, when n_active > K.
 */
int32_t npo_delta_step(int32_t M, int32_t K, int32_t* slot_map, int32_t* owner, const int32_t* S,
                       int32_t n_active, int32_t* d_in, int32_t* slot_in, int32_t* n_in,
                       int32_t* d_out, int32_t* n_out) {
    if (M <= 0 || K <= 0 || n_active < 0) return NPO_EINVAL;
    if (n_active > K) return NPO_ECAPACITY;
    char* in_s = (char*)calloc((size_t)M, 1);
    if (!in_s) return NPO_EINVAL;
    for (int32_t k = 0; k < n_active; ++k) {
        if (S[k] < 0 || S[k] >= M) { free(in_s); return NPO_EINVAL; }
        in_s[S[k]] = 1;
    }

    /* Step 2: set differences, ascending by neuron ID. */
    int32_t ni = 0, no = 0;
    for (int32_t i = 0; i < M; ++i) {
        int resident = slot_map[i] != -1;
        if (in_s[i] && !resident) d_in[ni++] = i;
        if (!in_s[i] && resident) d_out[no++] = i;
    }

    /* Step 3: release the outgoing neurons' slots. */
    for (int32_t k = 0; k < no; ++k) {
        int32_t i = d_out[k];
        owner[slot_map[i]] = -1;
        slot_map[i] = -1;
    }

    /* Step 4: the k-th incoming neuron takes the k-th free slot (ascending). */
    int32_t k = 0;
    for (int32_t s = 0; s < K && k < ni; ++s) {
        if (owner[s] == -1) {
            slot_in[k] = s;
            owner[s] = d_in[k];
            slot_map[d_in[k]] = s;
            ++k;
        }
    }
    free(in_s);
    *n_in = ni;
    *n_out = no;
    return NPO_OK;
}

/*
 * Residency window (LLM in a flash, section 3.1 "Windowing": weights of neurons that
 * were active for recent tokens stay resident, and only missing ones are loaded).
 * Computes the resident set R_t that the delta step then moves to (D_in = R_t \ R_{t-1},
 * D_out = R_{t-1} \ R_t), for token t, window k >= 1 and capacity K:
 *   R_t = S_t plus every resident neuron last active at token t - j, 1 <= j < k,
 *   taken from the most recent (j = 1) to the oldest and, within one j, by ascending ID,
 *   as long as |R_t| <= K. Neurons that left the buffer are never loaded back here.
 * k = 1 gives R_t = S_t (the exact rule of NeuroPrefetcher section 3.4).
 * last_t[i] is the last token at which neuron i was active (anything below t - k + 1 for
 * never). slot_map[i] >= 0 marks residency. Writes R_t ascending to R (capacity M) and
 * returns |R_t|; -2 when n > K (refused), -1 for invalid arguments.
 */
int32_t npo_window_target(int32_t M, int32_t K, int32_t k, int32_t t, const int32_t* last_t,
                          const int32_t* slot_map, const int32_t* S, int32_t n, int32_t* R) {
    if (M <= 0 || K <= 0 || k < 1 || n < 0) return -1;
    if (n > K) return -2;
    char* in_r = (char*)calloc((size_t)M, 1);
    if (!in_r) return -1;
    for (int32_t q = 0; q < n; ++q) {
        if (S[q] < 0 || S[q] >= M) { free(in_r); return -1; }
        in_r[S[q]] = 1;
    }
    int32_t room = K - n;
    for (int32_t j = 1; j < k && room > 0; ++j) {
        for (int32_t i = 0; i < M && room > 0; ++i) {
            if (in_r[i] || slot_map[i] < 0) continue;
            if (t - last_t[i] == j) {
                in_r[i] = 1;
                --room;
            }
        }
    }
    int32_t m = 0;
    for (int32_t i = 0; i < M; ++i)
        if (in_r[i]) R[m++] = i;
    free(in_r);
    return m;
}

/*
 * Frequency-weighted retention (DynamicInfer, key design 2, the hierarchical neuron cache: the
 * importance of neuron i is v = a + lambda * f, a = 1 when i is predicted active and f its
 * historical activation frequency, and the most important neurons are kept on the GPU,
 * replaced greedily by importance). Here every active neuron must be resident, so a = 1 ranks
 * first and the rest is ordered by f alone. f comes quantised: level[i] in [0, n_levels),
 * higher = more frequent. Computes R_t for capacity K:
 *   R_t = S_t plus resident neurons not in S_t, taken from the highest level down and, within
 *   one level, by ascending ID, as long as |R_t| <= K.
 * Neurons that are not resident are never loaded here (eviction only). With no room left
 * (|S_t| = K) or n_levels = 0 this is R_t = S_t, the exact rule of NeuroPrefetcher section 3.4.
 * Writes R_t ascending to R (capacity M) and returns |R_t|; -2 when n > K (refused), -1 for
 * invalid arguments (a level outside [0, n_levels) included).
 */
int32_t npo_level_target(int32_t M, int32_t K, int32_t n_levels, const uint8_t* level,
                         const int32_t* slot_map, const int32_t* S, int32_t n, int32_t* R) {
    if (M <= 0 || K <= 0 || n_levels < 0 || n < 0) return -1;
    for (int32_t i = 0; i < M && n_levels > 0; ++i)
        if (level[i] >= n_levels) return -1;
    if (n > K) return -2;
    char* in_r = (char*)calloc((size_t)M, 1);
    if (!in_r) return -1;
    for (int32_t q = 0; q < n; ++q) {
        if (S[q] < 0 || S[q] >= M) { free(in_r); return -1; }
        in_r[S[q]] = 1;
    }
    int32_t room = K - n;
    for (int32_t lv = n_levels - 1; lv >= 0 && room > 0; --lv) {
        for (int32_t i = 0; i < M && room > 0; ++i) {
            if (in_r[i] || slot_map[i] < 0 || level[i] != lv) continue;
            in_r[i] = 1;
            --room;
        }
    }
    int32_t m = 0;
    for (int32_t i = 0; i < M; ++i)
        if (in_r[i]) R[m++] = i;
    free(in_r);
    return m;
}

/*
 * Compacted buffer (LLM in a flash, section 3.3 "Optimized Data Management in DRAM": the
 * occupied rows always form the prefix 0 .. n-1 of the preallocated matrix; a removed neuron's
 * row is replaced by a row from the end of the occupied region, and incoming rows are appended
 * after it), with the set difference of NeuroPrefetcher section 3.4 deciding who leaves and
 * who comes. State: pos_map[M] (position of neuron i, -1 if absent), owner[K] (neuron at a
 * position, -1 past the end), *n_occ (rows in use). One step:
 *   1. D_in = S \ R and D_out = R \ S, ascending (R = the neurons in the buffer).
 *   2. Removal, one hole at a time in ascending position: rows at the end of the occupied
 *      region whose neuron leaves are dropped (the region shrinks); then the lowest position
 *      still held by a leaving neuron takes the last row of the region, which is recorded as a
 *      move (mv_src -> mv_dst) and the region shrinks by one. A leaving row is never moved.
 *   3. Appending: the k-th incoming neuron (ascending) goes to position n_keep + k, where
 *      n_keep = |R| - |D_out| is the region left after step 2.
 * Outputs (capacity K each): d_in / pos_in (n_in), d_out (n_out), mv_src / mv_dst (n_mv, in
 * ascending mv_dst). NPO_ECAPACITY, state untouched, when n_active > K.
 */
int32_t npo_compact_step(int32_t M, int32_t K, int32_t* pos_map, int32_t* owner, int32_t* n_occ,
                         const int32_t* S, int32_t n_active, int32_t* d_in, int32_t* pos_in,
                         int32_t* n_in, int32_t* d_out, int32_t* n_out, int32_t* mv_src,
                         int32_t* mv_dst, int32_t* n_mv) {
    if (M <= 0 || K <= 0 || n_active < 0) return NPO_EINVAL;
    if (n_active > K) return NPO_ECAPACITY;
    char* in_s = (char*)calloc((size_t)M, 1);
    char* leaving = (char*)calloc((size_t)M, 1);
    if (!in_s || !leaving) { free(in_s); free(leaving); return NPO_EINVAL; }
    for (int32_t k = 0; k < n_active; ++k) {
        if (S[k] < 0 || S[k] >= M) { free(in_s); free(leaving); return NPO_EINVAL; }
        in_s[S[k]] = 1;
    }
    /* Step 1 */
    int32_t ni = 0, no = 0;
    for (int32_t i = 0; i < M; ++i) {
        const int present = pos_map[i] != -1;
        if (in_s[i] && !present) d_in[ni++] = i;
        if (!in_s[i] && present) { d_out[no++] = i; leaving[i] = 1; }
    }
    /* Step 2 */
    int32_t n = *n_occ, nm = 0;
    for (;;) {
        while (n > 0 && leaving[owner[n - 1]]) {          /* drop leaving rows at the end */
            pos_map[owner[n - 1]] = -1;
            owner[n - 1] = -1;
            --n;
        }
        int32_t hole = -1;
        for (int32_t p = 0; p < n; ++p)
            if (leaving[owner[p]]) { hole = p; break; }
        if (hole < 0) break;
        const int32_t gone = owner[hole], mover = owner[n - 1];
        pos_map[gone] = -1;
        owner[hole] = mover;
        pos_map[mover] = hole;
        owner[n - 1] = -1;
        mv_src[nm] = n - 1;
        mv_dst[nm] = hole;
        ++nm;
        --n;
    }
    /* Step 3 */
    for (int32_t k = 0; k < ni; ++k) {
        pos_in[k] = n + k;
        owner[n + k] = d_in[k];
        pos_map[d_in[k]] = n + k;
    }
    *n_occ = n + ni;
    *n_in = ni;
    *n_out = no;
    *n_mv = nm;
    free(in_s);
    free(leaving);
    return NPO_OK;
}

/* The moves of one compact step: buf[mv_dst[k]] = buf[mv_src[k]] (sources and destinations
 * are disjoint, so the order does not matter). */
void npo_move_bundles(uint16_t* buf, int64_t bundle_elems, const int32_t* mv_src,
                      const int32_t* mv_dst, int32_t n_mv) {
    for (int32_t k = 0; k < n_mv; ++k)
        memcpy(buf + (int64_t)mv_dst[k] * bundle_elems, buf + (int64_t)mv_src[k] * bundle_elems,
               (size_t)bundle_elems * sizeof(uint16_t));
}

/* Ascending occupied slots (the slots whose rows the FFN reads); returns the count. */
int32_t npo_occupied_slots(int32_t K, const int32_t* owner, int32_t* slots) {
    int32_t n = 0;
    for (int32_t s = 0; s < K; ++s)
        if (owner[s] != -1) slots[n++] = s;
    return n;
}

/*
 * Step 4 bytes: buf[slot_in[k]] = bundle of neuron d_in[k], for k < n_in.
 * `store` holds the bundles of all neurons, `bundle_elems` bf16 values each.
 */
void npo_copy_bundles(uint16_t* buf, const uint16_t* store, int64_t bundle_elems,
                      const int32_t* d_in, const int32_t* slot_in, int32_t n_in) {
    for (int32_t k = 0; k < n_in; ++k) {
        memcpy(buf + (int64_t)slot_in[k] * bundle_elems, store + (int64_t)d_in[k] * bundle_elems,
               (size_t)bundle_elems * sizeof(uint16_t));
    }
}

static double npo_bf16_to_f64(uint16_t h) {
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)h << 16;
    return (double)v.f;
}

enum { NPO_ACT_RELU = 0, NPO_ACT_SILU = 1 };

/* The activation on the gate (or, non-gated, the up) dot product. */
static double npo_act(double g, int32_t act) {
    if (act == NPO_ACT_SILU) return g / (1.0 + exp(-g));
    return g > 0.0 ? g : 0.0;
}

/*
 * Sparse FFN in fp64. ids[k] (k < n) indexes the bundles in `store`
 * (bundle = n_rows rows of d bf16 values). n_rows = 3: [gate|up|down^T],
 * h = act(gate.x) * (up.x); n_rows = 2: [up|down^T], h = act(up.x).
 * y[d] = sum_k h_k * down_{ids[k]}, accumulated in the order given.
 * Returns NPO_EINVAL for an unsupported n_rows or activation.
 */
int32_t npo_sparse_ffn_act(const uint16_t* store, int32_t n_rows, int32_t d, const int32_t* ids,
                           int32_t n, const float* x, int32_t act, double* y) {
    if (n_rows != 2 && n_rows != 3) return NPO_EINVAL;
    if (act != NPO_ACT_RELU && act != NPO_ACT_SILU) return NPO_EINVAL;
    for (int32_t j = 0; j < d; ++j) y[j] = 0.0;
    for (int32_t k = 0; k < n; ++k) {
        const uint16_t* bundle = store + (int64_t)ids[k] * n_rows * d;
        const uint16_t* down = bundle + (int64_t)(n_rows - 1) * d;
        double h;
        if (n_rows == 3) {
            const uint16_t* gate = bundle;
            const uint16_t* up = bundle + d;
            double g = 0.0, u = 0.0;
            for (int32_t j = 0; j < d; ++j) {
                g += npo_bf16_to_f64(gate[j]) * (double)x[j];
                u += npo_bf16_to_f64(up[j]) * (double)x[j];
            }
            h = npo_act(g, act) * u;
        } else {
            const uint16_t* up = bundle;
            double u = 0.0;
            for (int32_t j = 0; j < d; ++j) u += npo_bf16_to_f64(up[j]) * (double)x[j];
            h = npo_act(u, act);
        }
        for (int32_t j = 0; j < d; ++j) y[j] += h * npo_bf16_to_f64(down[j]);
    }
    return NPO_OK;
}

/* The ReLU FFN (the benchmark's models). */
int32_t npo_sparse_ffn(const uint16_t* store, int32_t n_rows, int32_t d, const int32_t* ids,
                       int32_t n, const float* x, double* y) {
    return npo_sparse_ffn_act(store, n_rows, d, ids, n, x, NPO_ACT_RELU, y);
}
