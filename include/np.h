/*
 * np.h -- delta-prefetched sparse FFN for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The method: "NeuroPrefetcher: Storage-Aware Sparse LLM Inference via Delta
 * Prefetching" (Dhar et al.). For every sparse FFN layer and every decode
 * token at batch 1:
 *   1. the predicted active neuron set is decoded from the layer's gate and
 *      up centroid bitmasks (section 3.4; section 3.1: the centroid table is
 *      always resident);
 *   2. it is diffed against the rows resident in a fixed K_max-slot buffer
 *      (section 3.4, "by set difference");
 *   3. outgoing neurons release their slots and incoming neurons take freed
 *      slots, tracked by a slot map that is -1 for non-resident neurons
 *      (section 3.4; no compaction);
 *   4. the incoming neurons' [gate|up|down^T] bundles are scattered from the
 *      backing row store into their slots (section 3.5, the fused
 *      deinterleave-and-scatter, which there runs on a stream of its own so
 *      that it overlaps compute; in np_decode_step it runs inside the
 *      previous layer's FFN launch, on compute units of its own);
 *   5. the sparse FFN y = sum_{i in S} down_i * relu(gate_i . x) * (up_i . x)
 *      runs over the resident slots only (section 3.4: row i of gate, up and
 *      down^T per active neuron; the slot map locates the rows). A non-gated
 *      [up|down^T] bundle (LLM in a flash, section 3.2) gives
 *      y = sum_{i in S} down_i * relu(up_i . x).
 *
 * Conventions used by every call:
 *   - Every call returns np_status; NP_OK is 0. On any error the call has
 *     enqueued nothing and changed no state; np_last_error() returns a
 *     thread-local description of the last failure of the calling thread.
 *   - All argument, range, capacity and call-order checks run on the host,
 *     synchronously, before anything is enqueued. What only a kernel can
 *     detect is reported asynchronously: after a kernel of a layer raised
 *     error bits, the layer's enqueueing calls fail with NP_EDEVICE (see
 *     "Device-side errors" below).
 *   - "stream" arguments are hipStream_t handles passed as void*; NULL means
 *     the device's null stream. Compute calls are asynchronous on their
 *     stream; np_layer_read_* calls synchronize the layer's device.
 *   - A layer is not thread-safe, and its calls must be ordered (one stream,
 *     or the caller's events). Different layers may be driven from
 *     different threads.
 *   - Bit b of mask word w is neuron 64*w + b. Bundles are bf16 (raw 16-bit
 *     patterns), rows in the order gate, up, down^T (n_rows = 3) or up,
 *     down^T (n_rows = 2), d_model values per row, no padding.
 *   - The library owns every device allocation it makes; the caller owns the
 *     row store, x and y buffers and the streams.
 *
 * Limits checked at np_layer_create: d_model % 8 == 0 (128-bit rows),
 * 8 <= d_model <= 16384, 1 <= d_ff <= 65536, 1 <= k_max <= min(d_ff, 65536),
 * n_rows in {2, 3}, 1 <= n_centroids <= 65536, and the slot buffer
 * (k_max * n_rows * d_model * 2 bytes) below 4 GiB.
 */
#ifndef NP_H
#define NP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NP_OK = 0,
    NP_EINVAL = 1,     /* bad argument, shape, pointer or centroid ID            */
    NP_ECAPACITY = 2,  /* |S| > k_max for the requested centroid IDs             */
    NP_ENOMEM = 3,     /* device or host allocation failed                       */
    NP_EHIP = 4,       /* a HIP runtime call failed (text in np_last_error)      */
    NP_ESTATE = 5,     /* call-order violation (see np_delta_assign)             */
    NP_EDEVICE = 6     /* a kernel of the layer reported an inconsistency        */
} np_status;

/* How the two centroid masks combine into the active set (section 3.4 of the
 * paper intersects them; the Llama-shaped workloads use their union; SINGLE
 * uses one table for a non-gated FFN). */
typedef enum { NP_MASK_UNION = 0, NP_MASK_INTERSECT = 1, NP_MASK_SINGLE = 2 } np_mask_mode;

/* Activation on the gate (gated) or up (non-gated) dot product: ReLU (the
 * benchmark's gated-ReLU models; relu(0) = 0) or SiLU, g / (1 + exp(-g)), the
 * gate of the SwiGLU MLPs of section 3.4. Computed in fp32 on the GPU. */
typedef enum { NP_ACT_RELU = 0, NP_ACT_SILU = 1 } np_act;

typedef struct np_layer np_layer; /* opaque: one sparse FFN layer */

typedef struct np_layer_desc {
    int32_t d_model;     /* d: values per row                                    */
    int32_t d_ff;        /* M: neurons                                           */
    int32_t k_max;       /* K_max: resident slots                                */
    int32_t n_rows;      /* 3 = [gate|up|down^T], 2 = [up|down^T]                */
    int32_t n_centroids; /* C: masks per table                                   */
    int32_t mask_mode;   /* np_mask_mode                                         */
    int32_t act;         /* np_act                                               */
    int32_t device;      /* HIP device ordinal of the layer                      */
    /* host uint64 [n_tables][n_centroids][ceil(d_ff/64)], n_tables = 1 for
     * SINGLE else 2 (gate table, then up table). COPIED at create. Bits at
     * or above d_ff in the last word must be zero (NP_EINVAL otherwise). */
    const uint64_t* masks;
    /* bf16 [d_ff][n_rows][d_model], 16-byte aligned, BORROWED: the caller
     * keeps it alive and unchanged while the layer exists. It may be device
     * memory of `device` (the backing store sits in HBM) or pinned host
     * memory from hipHostMalloc (the scatter kernel then pulls the delta
     * bundles over the host link). Pageable host memory gives NP_EINVAL. */
    const void* row_store;
} np_layer_desc;

/* Sets up one sparse layer: the resident row buffer of k_max slots that
 * NeuroPrefetcher section 3.4 keeps per layer (allocated bf16
 * [k_max][n_rows][d_model], zero-filled), its slot map int32 [d_ff] (-1 for
 * a neuron that is not resident, section 3.4), the owner table int32
 * [k_max] (-1 = free slot), the resident and free bitsets, the delta lists
 * and the FFN scratch, and a device copy of the centroid masks (section 3.1
 * keeps the centroid table resident on the GPU). desc is read, not kept;
 * *out receives the layer, owned by the caller until np_layer_destroy.
 * Errors: NP_EINVAL (a limit above, a NULL or misaligned pointer, stray mask
 * bits, a row store that is neither device memory of `device` nor mapped
 * pinned host memory), NP_ENOMEM, NP_EHIP; *out is NULL on any error. */
np_status np_layer_create(const np_layer_desc* desc, np_layer** out);

/* Library infrastructure (no passage of the pages defines it): synchronizes
 * the layer's device, drops cached decode graphs that use the layer and
 * frees everything the layer allocated. The row store is the caller's and
 * is not touched. NP_EINVAL for NULL. */
np_status np_layer_destroy(np_layer* layer);

/* Back to the state np_layer_create leaves (empty buffer, zero-filled); the
 * next np_delta_assign is a cold start that fetches the whole active set
 * (section 3.4). Synchronous. */
np_status np_layer_reset(np_layer* layer);

/* Steps 1-3 for one layer (section 3.4). Builds S from mask gate_cid of the
 * gate table and up_cid of the up table (up_cid is ignored for SINGLE),
 * picks the new resident set R' (R' = S, or with a residency window or
 * frequency levels see np_layer_set_window and np_layer_set_levels), computes D_in = S \ R and D_out = R \ R' in
 * ascending neuron order, releases the slots of D_out, gives the i-th neuron
 * of D_in the i-th free slot in ascending slot order, updates the slot map
 * and owner table, and lists the slots of S in ascending slot order (the rows
 * the FFN reads). Then R = R'.
 * Errors: NP_EINVAL (cid out of range), NP_ECAPACITY (|S| > k_max; state
 * unchanged), NP_ESTATE (the previous assignment has not been scattered). */
np_status np_delta_assign(np_layer* layer, int32_t gate_cid, int32_t up_cid, void* stream);

/* Step 4 (section 3.5): copies the bundle of each neuron of the last D_in
 * from the row store into its assigned slot with 128-bit loads and stores.
 * Errors: NP_ESTATE unless np_delta_assign was the previous state change. */
np_status np_scatter_rows(np_layer* layer, void* stream);

/* Step 5: y[d_model] = sum over the resident (= active) slots of
 * down * act(gate . x) * (up . x), bf16 weights, fp32 arithmetic and
 * accumulation; the cross-workgroup reduction is set by np_layer_set_ffn_reduce.
 * x and y are fp32 [d_model], 16-byte aligned, not overlapping, in memory the layer's device
 * can access (its device memory, or mapped pinned host memory; anything else is NP_EINVAL
 * before any launch, as for np_decode_step's x and y). The
 * result is run-to-run identical with NP_REDUCE_ORDERED (np_layer_set_ffn_reduce).
 * Called right after np_delta_assign (no np_scatter_rows) with a row store in
 * device memory, it does step 4 itself: the bundles of the slots filled by
 * that assignment are read from the row store and written into their slots
 * by the same launch (read-through), with the same y and buffer contents.
 * The FFN addresses the row store with 32-bit offsets, so a device row store
 * above 4 GiB - 4096 bytes (d_ff * n_rows * d_model * 2) is instead scattered
 * into its slots by a launch of its own before the FFN; y and the buffer are
 * the same either way.
 * Errors: NP_ESTATE before the first np_delta_assign, or after an
 * unscattered assignment when the row store is host memory. */
np_status np_sparse_ffn(np_layer* layer, const float* x, float* y, void* stream);

/* As np_sparse_ffn, but y += FFN(x): the FFN output is added to what y holds
 * (the residual stream of a transformer block). Same state rules. */
np_status np_sparse_ffn_acc(np_layer* layer, const float* x, float* y, void* stream);

/* For callers that cannot allocate device memory while they run (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the FFN
 * step of np_sparse_ffn, with the same state rules and the same result, bit for
 * bit, as np_sparse_ffn with the ordered reduction (the default), but its
 * cross-workgroup exchange words live in a static per-device scratch of 2 MiB
 * (one word per active slot and one per partial sum of the launch) instead of
 * the layer's own. The call allocates and frees nothing (the layer itself is
 * created beforehand); it always uses the ordered reduction. The scratch is
 * part of the library, held on every device it runs on until the process
 * ends; every call on one device shares it, so calls that overlap on one
 * device (other streams, other host threads) race and give wrong results:
 * order them. Its address is taken when the device's first layer is created.
 * Errors: as np_sparse_ffn; NP_EINVAL (nothing enqueued) when the launch needs
 * more than 65,536 h words or 196,608 partial-sum words (launch shapes with
 * very many workgroups; np_sparse_ffn serves those); NP_EHIP if the scratch
 * has no device address on this device. */
np_status np_sparse_ffn_noalloc(np_layer* layer, const float* x, float* y, void* stream);

/* How the FFN's workgroups combine the partial sums of y (section 3.4 fixes
 * only the sum). NP_REDUCE_ORDERED (the default): the partial sums are
 * exchanged without atomics and added in a fixed order by one workgroup per
 * output tile, so y is bit-identical run to run. NP_REDUCE_ATOMIC (an
 * option): every workgroup adds its partial sums into y with fp32 atomics,
 * one cross-workgroup hop less; the order of the additions, and so the last
 * bits of y, can differ from run to run. np_sparse_ffn then clears y with
 * one extra launch; np_decode_step clears it inside its assign launch.
 * Synchronizes the device. */
typedef enum { NP_LAYOUT_SLOTS = 0, NP_LAYOUT_COMPACT = 1 } np_layout;
typedef enum { NP_REDUCE_ATOMIC = 0, NP_REDUCE_ORDERED = 1 } np_reduce;
np_status np_layer_set_ffn_reduce(np_layer* layer, int32_t mode);

/* One decode token over n_layers layers of one device with equal d_model
 * (sections 3.1, 3.4, 3.5): validates every layer's cids on the host (a
 * failure leaves every layer unchanged), then enqueues the token on
 * compute_stream: one launch assigns the deltas of all layers, then one
 * launch per layer runs that layer's FFN. A layer whose row store is device
 * memory has its FFN read the new bundles through from the store (as
 * np_sparse_ffn right after np_delta_assign; a device store above
 * 4 GiB - 4096 bytes is scattered by a launch of its own first). When every row store is
 * pinned host memory (and the layers share their FFN workgroup size), the
 * rest of the token is one launch per group of up to 64 layers, which
 * overlaps the host link with the FFNs (the prefetch of section 3.5): 24
 * workgroups copy every layer's new bundles, layer after layer, without a
 * break at layer boundaries, and each layer's FFN runs on the other compute
 * units as soon as its bundles are in place. Other pinned host stores:
 * layer 0's bundles are scattered by a launch of their own, and the FFN
 * launch of layer l also scatters layer l + 1's new bundles, on a few
 * compute units of their own, while the FFN runs on the rest.
 * copy_stream is used only for staged delta I/O (np_decode_set_staging):
 * then the staged layers' copies and scatters run there and layer l's FFN
 * waits only for layer l's, and copy_stream is joined back into
 * compute_stream at the end. cids: host int32 [n_layers][2] (gate, up).
 * x, y: device fp32 [n_layers][d_model]. Every layer must be in the fresh
 * or scattered state (NP_ESTATE otherwise); after NP_EHIP the layers need
 * np_layer_reset. */
np_status np_decode_step(np_layer* const* layers, int32_t n_layers, const int32_t* cids,
                         const float* x, float* y, void* compute_stream, void* copy_stream);

/* Process-wide switch for np_decode_step. 0 (the default): the launches are
 * issued one by one. 1: the first call for a given (layer set, compute
 * stream, copy stream) captures the step's launches into a HIP graph; every
 * call then writes that token's centroid IDs, x and y pointers into a small
 * device parameter block with one kernel launch and replays the graph on
 * compute_stream, so a token costs two host calls (for callers whose host
 * thread is the bottleneck; on the GPU the extra parameter launch can make a
 * step slightly longer). The graph is rebuilt when a
 * layer is reset, reshaped or destroyed. Streams must be non-NULL for the
 * graph path (otherwise, and if capture fails, the launches are issued one by
 * one). Results are the same either way. */
np_status np_decode_use_graphs(int32_t enable);

/* Delta I/O of np_decode_step for row stores in pinned host memory.
 * bytes = 0 (the default): zero-copy pull, the scatter kernel reads the
 * incoming bundles over the host link. bytes > 0: the I/O shape of
 * NeuroPrefetcher section 3.5 -- the host copies each layer's incoming
 * bundles, in ascending neuron order and with adjacent neurons merged into
 * one copy, into a pinned staging buffer of `bytes` (two of them, used in
 * turn), the DMA engine copies the staging to device memory and a kernel
 * places each bundle in its slot; a delta larger than the staging goes in
 * several chunks. threads host threads share each gather (0: min(8, cores)).
 * Applies to layers without a window or frequency levels (their delta is
 * known on the host); others keep the zero-copy pull. A staged
 * np_decode_step returns once every gather is done, and is never replayed
 * from a graph. 0 <= bytes <= 1 GiB (a chunk must hold one bundle, else
 * np_decode_step fails with NP_EINVAL), 0 <= threads <= 64. Waits for the
 * copies of the staging buffers it replaces. Process-wide setting. */
np_status np_decode_set_staging(int64_t bytes, int32_t threads);

/* Inspection of the state NeuroPrefetcher section 3.4 defines: the slot map
 * (-1 for a neuron without a slot), the delta lists of the last set
 * difference (D_in = S \ R and D_out = R \ S, ascending) and the slots the
 * incoming neurons took. Synchronizes the layer's device, then copies the
 * current state to host buffers (any pointer may be NULL): slot_map int32 [d_ff], owner int32
 * [k_max], d_in / slot_in / d_out int32 [k_max] (lists of the last
 * assignment), act_slots int32 [k_max] (ascending slots of S; with window 1
 * these are all occupied slots), counts
 * int32 [4] = {n_in, n_out, n_active, device error bits}.
 * Returns NP_EDEVICE if a kernel of this layer reported an inconsistency
 * (nonzero error bits; the data is still copied). */
np_status np_layer_read_state(const np_layer* layer, int32_t* slot_map, int32_t* owner,
                              int32_t* d_in, int32_t* slot_in, int32_t* d_out,
                              int32_t* act_slots, int32_t* counts);

/* Inspection of the resident buffer (NeuroPrefetcher section 3.4: the rows of
 * the active neurons at the slots the slot map gives; section 3.5: one
 * neuron-centric [gate|up|down^T] record per neuron). Synchronizes, then
 * copies the bundles of the given slots (each < k_max) into dst (host,
 * n * n_rows * d_model bf16, in bundle order whatever the buffer
 * arrangement). slots == NULL with n == k_max copies the whole buffer,
 * stale rows of freed slots included. NP_EINVAL for a slot out of range
 * (nothing copied). */
np_status np_layer_read_rows(const np_layer* layer, const int32_t* slots, int32_t n, void* dst);

/* Host-side view: out[0..5] = {d_model, d_ff, k_max, n_rows, n_active of the
 * last accepted assignment, n_in of the last accepted assignment}. */
np_status np_layer_info(const np_layer* layer, int32_t* out6);

/* Running totals since create/reset: out2[0] = sum of |S| and out2[1] = sum
 * of |D_in| over every accepted assignment (bundles read by the FFN and
 * bundles written by the scatter, in units of one bundle). Host-side and
 * non-blocking with window 1 and no levels; otherwise |D_in| is known on the
 * device only and the call synchronizes the layer's device. */
np_status np_layer_counters(const np_layer* layer, int64_t* out2);

/* Residency window (LLM in a flash, section 3.1 "Windowing"): besides S, the
 * buffer keeps the resident neurons that were active in the last window - 1
 * tokens, the most recently active first and by ascending neuron ID within
 * one token, as long as at most k_max neurons are resident. Kept neurons
 * cost no transfer when they become active again; a neuron that left is only
 * loaded again when it is active. window = 1 (the default) is the exact rule
 * of section 3.4: the buffer holds S. 1 <= window <= 16. Only before the
 * first np_delta_assign after create or reset (NP_ESTATE otherwise).
 * Exclusive with frequency levels (np_layer_set_levels; NP_EINVAL).
 * Synchronizes the layer's device. With window > 1, np_layer_info's n_in and
 * np_layer_counters' |D_in| are read back from the device. */
np_status np_layer_set_window(np_layer* layer, int32_t window);

/* Retention by frequency level (DynamicInfer paper notes, key design 2, the
 * hierarchical neuron cache: importance a + lambda * f, a = 1 for a
 * predicted-active neuron, f its historical activation frequency). Every
 * active neuron is resident, so only the neurons outside S are ranked, by
 * f: besides S the buffer keeps resident neurons by descending level, then
 * ascending neuron ID, as long as at most k_max neurons are resident; a
 * neuron that left is only loaded again when it is active. level is host
 * uint8 [d_ff], each value < n_levels (higher = more frequent), the
 * caller's quantisation of offline activation frequencies; it is copied.
 * n_levels = 0 switches the retention off (level may be NULL): the buffer
 * holds exactly S again. 0 <= n_levels <= 16. Exclusive with a window > 1
 * (NP_EINVAL). Only before the first np_delta_assign after create or reset
 * (NP_ESTATE otherwise). Synchronizes the layer's device. With n_levels > 0,
 * np_layer_info's n_in and np_layer_counters' |D_in| are read back from
 * the device. */
np_status np_layer_set_levels(np_layer* layer, int32_t n_levels, const uint8_t* level);

/* Buffer layout. NP_LAYOUT_SLOTS (the default; NeuroPrefetcher section 3.4):
 * the slot map, incoming neurons take the lowest free slots, no compaction.
 * NP_LAYOUT_COMPACT (LLM in a flash, section 3.3 "Optimized Data Management
 * in DRAM"): the rows of S always occupy positions 0 .. |S|-1; with
 * n_keep = |R| - |D_out|, each leaving row below n_keep (ascending) is
 * replaced by the last staying row of the region (a move, copied on the
 * device right after the assignment, before any new row is written), and
 * the k-th incoming neuron (ascending) is appended at n_keep + k. The slot
 * map, owner table and slot_in of np_layer_read_state then hold positions.
 * Needs window 1 and no frequency levels (NP_EINVAL). Only before the first
 * np_delta_assign after create or reset (NP_ESTATE). Synchronizes the
 * layer's device. */
np_status np_layer_set_layout(np_layer* layer, int32_t layout);

/* The moves of the last assignment of a compacted layer: src[k] -> dst[k]
 * (positions, ascending dst), *n_moves of them (capacity k_max each; 0 for
 * the slot layout; src or dst may be NULL). Synchronizes the layer's
 * device. */
np_status np_layer_read_moves(const np_layer* layer, int32_t* src, int32_t* dst, int32_t* n_moves);

/* Arrangement of the slot buffer (NeuroPrefetcher section 3.5 keeps the
 * resident rows in planar per-projection buffers). planar = 0 (the
 * default): one interleaved bundle [gate|up|down^T] per slot, buffer bf16
 * [k_max][n_rows][d_model]. planar = 1: one buffer per row kind, bf16
 * [n_rows][k_max][d_model], so slot s's row r is plane r, row s; the scatter
 * kernels and the FFN's read-through then split each bundle into its
 * planes. The same bytes are read by the FFN either way; np_layer_read_rows
 * returns bundles in both. Only before the first np_delta_assign after
 * create or reset (NP_ESTATE). Synchronizes the layer's device. */
np_status np_layer_set_planar(np_layer* layer, int32_t planar);

/* FFN launch shape of this layer: about slots_per_wg active slots per
 * workgroup for the gate/up phase (1..16; the default, -1, sizes the grid to
 * one workgroup per compute unit), tile_cols output
 * columns per workgroup for the down phase (8 * a power of two, 64..1024,
 * default 256) and threads per workgroup (256, 512 or 1024; default by
 * d_model; tile_cols must not exceed threads). 0 keeps the current value;
 * slots_per_wg = -1 restores the per-compute-unit default.
 * Synchronizes the device. The shape
 * changes speed and the fp32 summation order, not what is computed.
 * NP_EINVAL if the shape cannot cover k_max active slots. */
np_status np_layer_set_ffn_shape(np_layer* layer, int32_t slots_per_wg, int32_t tile_cols, int32_t threads);

/* Library infrastructure (no passage of the pages defines it): the calling
 * thread's text of its last failed call ("" if none). The pointer stays
 * valid until that thread's next failing call. */
const char* np_last_error(void);

/* Device-side errors. A kernel that finds an inconsistency (a list entry out of range, no
 * free slot, a wait that hit its iteration limit, host and device counts that differ) ORs
 * error bits into the layer's device counts and stores them into a pinned host word of the
 * layer, without stopping. From then on, every call that enqueues work for the layer
 * (np_delta_assign, np_scatter_rows, np_sparse_ffn, np_sparse_ffn_acc, np_decode_step) fails
 * with NP_EDEVICE before enqueuing anything, and np_layer_read_state returns the bits (with
 * NP_EDEVICE); np_layer_reset clears them. The host word is read without synchronizing, so the
 * report comes at the first such call after the kernel's store reached host memory.
 *
 * np_layer_raise_error makes the layer raise `bits` (> 0) through that same device path, as a
 * kernel on `stream` would: for testing the reporting without a failing kernel. */
np_status np_layer_raise_error(np_layer* layer, int32_t bits, void* stream);

/* ---- measurement probes (roofline denominators and counter scaling) ---- */

/* Streaming read of `bytes` (multiple of 16) at src (device or pinned host);
 * writes one float per workgroup into sink (device, >= 65536 floats) so the
 * loads are not dead. */
np_status np_probe_read(const void* src, int64_t bytes, float* sink, void* stream);

/* The same streaming read over n_srcs buffers of `bytes` each (srcs: host array of device
 * pointers, each 16-byte aligned), launched `passes` times over the whole set, back to back on
 * `stream` from the library's own loop: the per-launch cost of a plain read of that many bytes
 * without host launch overhead. Rotating over more bytes than the GPU's last-level cache keeps
 * every launch a read from HBM. 1 <= n_srcs <= 4096, 1 <= passes <= 1000; all checks run
 * before the first launch (NP_EINVAL). */
np_status np_probe_read_set(const void* const* srcs, int32_t n_srcs, int64_t bytes, int32_t passes, float* sink,
                            void* stream);

/* Plain 128-bit copy kernel, bytes a multiple of 16, no overlap. */
np_status np_probe_copy(void* dst, const void* src, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NP_H */
