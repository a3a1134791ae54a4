/*
 * moe_cache.h -- C ABI of libmoecache.so: one routed-expert MoE layer forward
 * on an AMD Instinct MI355X (gfx950), with expert weights reached through a
 * GPU-resident LRU cache of whole (layer, expert) entries.
 *
 * What the FreeToken pages state, and this library implements:
 *  - each token activates a subset of the experts; DeepSeek-V4-Flash picks 6
 *    of 256 routed experts per layer (RTX-4090 page, "How the MoE memory
 *    hierarchy works"); the runtime decides which weights stay on the GPU and
 *    which stay in host memory (llama page, "Official project overview").
 *  - the host holds the full routed-expert pool as ground truth; the GPU holds
 *    a shared cache of complete (layer, expert) entries under the same logical
 *    mapping (RTX-4090 page, "How the MoE memory hierarchy works"; benchmark
 *    page, runtime-tier table).
 *  - decode keeps one global LRU expert cache across layers and tokens; misses
 *    move over PCIe into the GPU cache (llama page, "Official project
 *    overview"; benchmark page, "How FreeToken serves large MoE models").
 *  - prefill streams whole layers double-buffered: the next layer's experts
 *    cross PCIe while the current layer computes (same sections).
 *  - device-resident control data keeps routing-dependent decisions
 *    compatible with captured graph execution (benchmark page, feature card
 *    "graph compatibility").
 * The layer math (softmax top-k gate, SwiGLU experts, weighted combine) is
 * not on the pages; see the readings listed in the design notes.
 *
 * Conventions for every entry point:
 *  - Returns an int status: MOE_OK or a negative MOE_E* code.  Nothing throws.
 *  - Host-detected errors return before anything is enqueued.
 *  - All work is asynchronous on the caller's stream; the library allocates
 *    nothing and the caller owns all memory.  The only global state is the
 *    fixed scratch array of moe_expert_ffn_noalloc (one per GPU, part of the
 *    loaded code object) and the cached device address of each GPU's copy.
 *  - Device pointers must be 16-byte aligned.  Errors found on the device are
 *    written to a caller-provided int32 device status word, sticky: the first
 *    error code is kept (compare-and-swap from 0); the caller reads it after a
 *    synchronisation.  This keeps the calls graph-capturable.
 *  - Calls sharing a cache descriptor or workspace must be ordered on one
 *    stream (not thread-safe on one descriptor).
 *  - Capture-safe (no host sync, no allocation, launch shape depends only on
 *    scalar arguments): every call except cache_fill, whose copy count is
 *    data-dependent and read on the host; cache_fill_device is its
 *    capture-safe counterpart.
 *
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 16), T >= 0 (T = 0 is a no-op),
 * T*k < 2^31, d and f positive multiples of 64.
 */
#ifndef MOE_CACHE_H
#define MOE_CACHE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* null pointer, bad size, limit exceeded */
#define MOE_EUNSUPPORTED (-2) /* dtype combination not implemented */
#define MOE_EHIP (-3)         /* a HIP launch or copy failed */
#define MOE_ECAPACITY (-4)    /* more unique experts requested than cache slots */
#define MOE_ERANGE (-5)       /* id, layer or slot out of range; stale cache slot */
#define MOE_ETOOBIG (-6)      /* larger than a fixed library limit (no-allocation scratch) */
#define MOE_ETIMEOUT (-7)     /* a bounded device wait gave up (see moe_decode_token) */

#define MOE_F32 0   /* IEEE binary32 */
#define MOE_BF16 1  /* bfloat16 (upper half of binary32) */
#define MOE_MXFP4 2 /* expert weights only: OCP MX FP4, see moe_entry_bytes */

/* Static text for a status code. */
const char* moe_strerror(int status);

/* ABI version of this header (increments on incompatible change). */
int moe_abi_version(void);

/* Router logits (helper for workloads that start from activations):
 * logits[t][e] = sum_c x[t][c] * w_router[e][c], fp32 accumulate.
 * x [T][d] and w_router [E][d] row-major in `dtype` (MOE_F32 only);
 * logits [T][E] fp32.  The router itself is standard MoE practice: every
 * token scores every routed expert before the top-k choice (RTX-4090 page,
 * "How the MoE memory hierarchy works"). */
int moe_router_logits(const void* x, const void* w_router, int dtype, int T, int d, int E,
                      float* logits, hipStream_t stream);

/* Top-k routing with a softmax gate over the selected logits (RTX-4090 page,
 * "How the MoE memory hierarchy works": a token selects 6 of 256 experts).
 * logits [T][E] fp32 row-major (device).  Writes topk_ids [T][k] int32: the k
 * experts with the largest logits, in descending logit order, equal logits
 * (compared by value, -0 == +0) ordered by ascending expert id; and
 * topk_w [T][k] fp32 = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k
 * selected logits.  NaN logits are not supported (unchecked). */
int moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
              hipStream_t stream);

/* Workspace bytes moe_permute needs for (T, k, E). */
size_t moe_permute_workspace_bytes(int T, int k, int E);

/* Grouping tokens by expert: a stable counting sort of the T*k flat
 * assignments a = t*k + j by expert id (the grouping step before the expert
 * contraction; the pages describe experts running on the GPU for the tokens
 * routed to them: RTX-4090 page, component table).
 * topk_ids [T*k] int32 (device).  Writes counts [E], offsets [E+1] (exclusive
 * prefix of counts, offsets[E] = T*k), perm [T*k] (sorted position p -> a,
 * experts ascending, (t, j) order inside an expert) and inv [T*k] (a -> p).
 * ws: device workspace of at least moe_permute_workspace_bytes(T, k, E).
 * An id outside [0, E) sets *status = MOE_ERANGE (if status is not NULL) and
 * leaves the outputs undefined.  Results are deterministic (no atomics decide
 * an order). */
int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, int32_t* status,
                hipStream_t stream);

/* moe_route followed by moe_permute, with the same results (both steps as defined
 * above).  For T <= 16 both run in one launch (one workgroup routes the tokens
 * and groups the assignments), which saves a kernel boundary on the decode
 * path; larger T makes the two calls.  ws / ws_bytes as for moe_permute (not
 * touched by the one-launch form); status as for moe_permute. */
int moe_route_permute(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                      size_t ws_bytes, int32_t* status, hipStream_t stream);

/* Entry layout of one (layer, expert) cache entry, in w_dtype elements:
 *   [ W_gate: f rows x d ][ W_up: f rows x d ][ W_down: d rows x f ]
 * every matrix row-major with the contraction index contiguous (W_gate row i
 * holds the d input weights of gate unit i; W_down row o holds the f weights
 * of output channel o).  One entry is 3*d*f elements; entries sit at
 * arena + slot * entry_stride bytes (entry_stride >= 3*d*f*elem, multiple of
 * 16).  The same layout is used by the host pool, the device cache arena and
 * the streaming buffers, so a fill is one contiguous copy. */

/* Bytes of one (layer, expert) entry with weights in w_dtype (0 for an unknown type).
 * MOE_F32 / MOE_BF16: 3*d*f elements, [W_gate f x d][W_up f x d][W_down d x f].
 * MOE_MXFP4 (the pages deploy DeepSeek-V4-Flash routed experts in MXFP4:
 * benchmark page, "FreeToken benchmark results", model table; format: OCP
 * Microscaling Formats (MX) v1.0): every row of K contraction elements is K/32
 * blocks of 32 FP4 E2M1 codes sharing one E8M0 scale 2^(s - 127); a block's 16
 * code bytes hold element 2j in the low nibble of byte j, element 2j+1 in the
 * high nibble.  Entry bytes:
 *   [codes W_gate][codes W_up][codes W_down][scales W_gate][scales W_up][scales W_down]
 * with f*d/2 code bytes and f*d/32 scale bytes per matrix, = 3*d*f*17/32 in all
 * (13.4 MB at d=4096, f=2048, vs 50.3 MB in bf16).  Each R x K matrix is stored
 * in tiles of 16 rows x 128 elements, so that one 1 KB read is one tile: rows
 * 16*rt .. 16*rt+15 start at byte 8*K*rt of the matrix's codes (K/2*rt of its
 * scales); tile kt of that strip at +1024*kt (+64*kt), the strip's last tile
 * holding the K mod 128 elements left when K is not a multiple of 128; inside a
 * tile, slot l = 16*q + i (16 code bytes at 16*l, the scale byte at l) is row i
 * of the strip, elements 32*q .. 32*q+31 of the tile.  So block b of row r has
 * its codes at 8*K*(r/16) + 1024*(b/4) + 16*(16*(b%4) + r%16) and its scale at
 * K/2*(r/16) + 64*(b/4) + 16*(b%4) + r%16. */
size_t moe_entry_bytes(int d, int f, int w_dtype);

/* Workspace bytes for moe_expert_ffn: the SwiGLU intermediate [T*k][f] (2 bytes per unit,
 * 4 with MOE_F32 activations), and up to 16 tokens with MOE_BF16 activations 4 bytes per
 * unit, room for the one-launch MXFP4 path (see moe_expert_ffn's ws). */
size_t moe_expert_ffn_workspace_bytes(int T, int k, int f, int act_dtype);

#define MOE_PATH_AUTO 0 /* chosen from T*k/E on the host: the grouped GEMM above 2 rows per \
                           expert on average for bf16 weights, above 8 for MXFP4 */
#define MOE_PATH_GEMV 1 /* weight-streaming skinny path (decode-shaped counts) */
#define MOE_PATH_GEMM 2 /* LDS-tiled grouped GEMM (prefill-shaped counts) */

/* Expert SwiGLU FFNs over the grouped rows (RTX-4090 page, component table:
 * the GPU executes the experts it holds; the FFN form is a reading).
 * For every expert e with n_e = offsets[e+1] - offsets[e] > 0 (and
 * expert_mask[e] != 0 when expert_mask is not NULL), for p in
 * [offsets[e], offsets[e+1]): with X = x[perm[p] / k],
 *   h = SiLU(X W_gate^T) * (X W_up^T),  y_perm[p] = h W_down^T,
 * SiLU(z) = z / (1 + exp(-z)), fp32 accumulation.
 *  x: [T][d] in act_dtype; weights of e at arena + expert_slot[e]*entry_stride
 *  (expert_slot NULL = identity slots); y_perm [T*k][d] in y_dtype.
 *  MOE_F32 weights need MOE_F32 activations and y (fp32 arithmetic end to
 *  end); MOE_BF16 weights need MOE_BF16 activations, y fp32 or bf16, and
 *  round h to bf16 before the down projection.  MOE_MXFP4 weights (entry
 *  layout under moe_entry_bytes) need MOE_BF16 activations; each weight is its
 *  exact value (E2M1 value x block scale), the rest as for MOE_BF16.  MXFP4 runs
 *  on both paths (the weight-streaming one for d, f <= 8128).  With MOE_BF16
 *  weights the GEMM path needs T*d, T*k*f and 3*d*f each <= 2^32 (it keeps
 *  element offsets in 32 bits): MOE_PATH_GEMM past that returns
 *  MOE_EUNSUPPORTED, MOE_PATH_AUTO takes the weight-streaming kernels.
 *  slot_key (nullable, device, [S]): when given, a slot whose key is not
 *  key_base + e, or a negative slot, sets *status = MOE_ERANGE and that
 *  expert's rows are not written (stale-cache detection).
 *  ws: 16-byte aligned, at least T*k*f*2 bytes (4 with MOE_F32 activations), or
 *  MOE_EINVAL.  With MOE_MXFP4 weights on the weight-streaming path, T <= 16,
 *  min(E, T*k)*f >= 65536 and at least T*k*f*4 bytes (what
 *  moe_expert_ffn_workspace_bytes returns there), both projections run in one launch that
 *  exchanges h through tagged entries in ws (zeroed by a small kernel first); the results
 *  are bit-identical to the two-launch form a smaller ws takes.  A bounded wait inside that
 *  launch that gives up sets *status = MOE_ETIMEOUT (y_perm is then undefined). */
int moe_expert_ffn(const void* x, int act_dtype, const int32_t* perm, const int32_t* offsets,
                   int T, int k, int E, int d, int f, const int32_t* expert_slot,
                   const void* arena, size_t entry_stride, int w_dtype,
                   const uint8_t* expert_mask, const int32_t* slot_key, int key_base, void* ws,
                   size_t ws_bytes, void* y_perm, int y_dtype, int path, int32_t* status,
                   hipStream_t stream);

/* moe_expert_ffn without a workspace argument, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The SwiGLU intermediate lives in a fixed library-owned device array of
 * moe_expert_ffn_noalloc_max_bytes() bytes (8 MiB) on each GPU, held from the library's load
 * until the process ends; nothing is allocated by the call (its first call on a device looks
 * up that device's array address once).  Every other argument, result and error is as for
 * moe_expert_ffn, which it calls with the array as ws (so calls of up to 16 tokens whose
 * tagged entries fit take the one-launch MXFP4 path).  A call whose intermediate (T*k*f*2
 * bytes, 4 with MOE_F32 activations) exceeds the array returns MOE_ETOOBIG before anything
 * is enqueued.  All calls on
 * one GPU share its array and each overwrites it: calls that may overlap in time on one GPU
 * (different streams, or different host threads) race and give undefined results; order them
 * on one stream.  No part of the array needs to start at zero. */
int moe_expert_ffn_noalloc(const void* x, int act_dtype, const int32_t* perm,
                           const int32_t* offsets, int T, int k, int E, int d, int f,
                           const int32_t* expert_slot, const void* arena, size_t entry_stride,
                           int w_dtype, const uint8_t* expert_mask, const int32_t* slot_key,
                           int key_base, void* y_perm, int y_dtype, int path, int32_t* status,
                           hipStream_t stream);

/* Size in bytes of moe_expert_ffn_noalloc's fixed scratch array (its largest intermediate). */
size_t moe_expert_ffn_noalloc_max_bytes(void);

/* Weighted combine: out[t][:] = sum_{j=0..k-1} topk_w[t][j] * y_perm[inv[t*k+j]][:],
 * j ascending, fp32, a gather (no atomics, deterministic).  y_perm [T*k][d]
 * in y_dtype (MOE_F32 or MOE_BF16), out [T][d] fp32.
 * The pages name no combine rule; this is a reading: each token's output is
 * the gate-weighted sum of the outputs of the experts it selected (the step
 * that completes a token once its chosen experts have run, RTX-4090 page,
 * "How the MoE memory hierarchy works": a token activates only its selected
 * experts), with the gate weights of moe_route. */
int moe_combine(const void* y_perm, int y_dtype, const int32_t* inv, const float* topk_w, int T,
                int k, int d, float* out, hipStream_t stream);

/* Workspace bytes moe_decode_token needs: a 256-byte header (the launch epoch
 * word), then the SwiGLU intermediate as 8-byte entries (up to two bf16 values
 * and the epoch of the launch that wrote them), k*f entries at most. */
size_t moe_decode_token_workspace_bytes(int k, int f);

/* One token's routed-MoE layer in a single launch: moe_route_permute,
 * moe_expert_ffn and moe_combine for T = 1 (a decode step of one sequence:
 * the token activates only its k selected experts, RTX-4090 page, "How the
 * MoE memory hierarchy works"), with MOE_BF16 weights and activations.
 *   logits [E] fp32: the token is routed as by moe_route (top-k, softmax over
 *   the k winners) and the ids and weights are written to topk_ids [k] and
 *   topk_w [k] when those are not NULL.  logits NULL: topk_ids and topk_w
 *   are inputs instead (ids routed earlier, e.g. before a cache lookup).
 *   x [d] bf16; the weights of expert e at arena + expert_slot[e]*entry_stride
 *   (expert_slot NULL = identity), laid out as for moe_expert_ffn.
 *   out [d] fp32: out = sum_{j ascending} topk_w[j] * FFN_{topk_ids[j]}(x), the
 *   FFN as in moe_expert_ffn with h rounded to bf16 and each expert's output
 *   kept in fp32; bit-identical to moe_route_permute + moe_expert_ffn
 *   (y_dtype MOE_F32) + moe_combine on the same device.
 *   An id outside [0, E), a negative slot, or (slot_key not NULL) a slot
 *   whose key is not key_base + e sets *status = MOE_ERANGE and leaves that
 *   expert's term out of the sum.
 *   ws: moe_decode_token_workspace_bytes(k, f) bytes, 16-byte aligned,
 *   zero-filled by the caller before its first use and not written by the
 *   caller afterwards (each call advances the epoch word at its head by one;
 *   nothing needs clearing between calls or graph replays).  Calls that share
 *   a workspace must not overlap in time (order them on one stream).
 *   The launch is one grid of workgroups, no more than fit on the GPU at once,
 *   that run all gate/up work before any down work; a workgroup's first down
 *   item waits (bounded) until every workgroup has finished its gate/up
 *   work.  That needs all of them resident together: a call that overlaps
 *   another moe_decode_token call on the same GPU, or a launch that holds the
 *   compute units and never finishes, can make the wait give up, which sets
 *   *status = MOE_ETIMEOUT (the result is then undefined).
 * Shapes: d, f multiples of 64, d <= 8192, f <= 8192 and (d + k*f)*2 <= 65536
 * bytes (x and h are held in LDS), else MOE_EUNSUPPORTED; other weight types
 * MOE_EUNSUPPORTED.  Argument errors return before anything is enqueued. */
int moe_decode_token(const float* logits, const void* x, int E, int k, int d, int f,
                     const int32_t* expert_slot, const void* arena, size_t entry_stride,
                     int w_dtype, const int32_t* slot_key, int key_base, int32_t* topk_ids,
                     float* topk_w, void* ws, size_t ws_bytes, float* out, int32_t* status,
                     hipStream_t stream);

/* ---- global LRU expert cache over (layer, expert) entries ------------------ */

/* Cache descriptor.  All pointers except host_pool are device memory owned by
 * the caller.  Key of (layer, e) is layer*E + e.
 *   slot_of [L*E] int32: slot holding a key, -1 = absent
 *   key_of  [S]   int32: key in a slot, -1 = empty
 *   stamp   [S]   int64: last use (clock value), 0 = never
 *   clock   [1]   int64: number of completed lookups
 *   stats   [4]   int64: accesses, hits, misses, fill bytes (accumulated)
 *   status  [1]   int32: sticky device error word
 *   arena: S entries of entry_bytes each (device)
 *   host_pool: pinned host memory holding pool_entries whole entries,
 *   layer-major (entry (layer, e) at byte (layer*E + e) * entry_bytes): the
 *   ground-truth copy of every routed expert (vram page, opening section).
 *   pool_entries: entries host_pool holds (normally L*E).  A fill of
 *   (layer, e) with layer*E + e >= pool_entries is out of range, so a record
 *   can never read past a short pool; 0 when the cache has no pool. */
typedef struct {
  int32_t L, E, S;
  int32_t pool_entries;
  size_t entry_bytes;
  int32_t* slot_of;
  int32_t* key_of;
  int64_t* stamp;
  int64_t* clock;
  int64_t* stats;
  int32_t* status;
  void* arena;
  const void* host_pool;
} moe_cache_t;

/* One miss fill: copy pool entry (layer, expert) into slot; evicted_key = the
 * key the slot held before (-1 if it was empty). */
typedef struct {
  int32_t slot, layer, expert, evicted_key;
} moe_fill_t;

/* Empty cache: slot_of = key_of = -1, stamp = clock = stats = 0, status = 0.
 * The pages describe the GPU cache as filled by recent routing rather than fixed
 * at start-up (RTX-4090 page, "How the MoE memory hierarchy works"; llama page,
 * "Official project overview"); the reading taken here is that it starts empty
 * (cold) and every entry arrives through a miss fill.
 * Runs a fill kernel (no memset nodes), so it may be captured.  1 <= S <= 4096
 * (the lookup sorts one key per slot in LDS). */
int cache_init(const moe_cache_t* cache, hipStream_t stream);

/* One lookup/update of the global LRU for `layer` with the T*k requested ids
 * (pages: shared LRU of whole (layer, expert) entries, recent routing decides
 * residency; RTX-4090 page, "How the MoE memory hierarchy works").  One
 * workgroup on the device:
 *   t = clock + 1; U = sorted unique requested ids (a repeat is one access);
 *   if |U| > S: *status = MOE_ECAPACITY, *n_fills = 0, nothing else changes;
 *   every resident e in U gets stamp t (hit);
 *   misses (U minus hits, ascending id) take the slots with stamp < t in
 *   ascending (stamp, slot) order (empty slots first; entries used in this
 *   call are never evicted by it); each evicts the slot's old key;
 *   fills[i] = (slot, layer, expert, evicted key) in miss order; clock = t.
 * expert_slot [E] (device): slot of each requested expert, -1 for the rest.
 * fills: device array of at least min(E, T*k) records; n_fills: device int32.
 * An id outside [0, E) sets MOE_ERANGE and changes nothing. */
int cache_lookup_update(const moe_cache_t* cache, int layer, const int32_t* topk_ids, int T, int k,
                        int32_t* expert_slot, moe_fill_t* fills, int32_t* n_fills,
                        hipStream_t stream);

/* cache_lookup_update with the misses split between PCIe fills and host
 * execution (the q-star policy: the runtime measures host-side expert
 * throughput and pinned PCIe bandwidth and decides from them how many misses
 * move to the GPU and how many run on the CPU; benchmark page, "How FreeToken
 * serves large MoE models", its runtime-tier table and "adaptive cache miss"
 * card; RTX-4090 page, "Setup and tuning workflow", "Measure the system").
 * With m misses this call fills q* of them, q* minimising
 * max(q * host_mbps, (m - q) * pcie_mbps) over q = 0..m (the two concurrent
 * paths' times for entries of equal size), ties to the larger q: the first q*
 * misses in ascending id are handled exactly as cache_lookup_update handles
 * misses; the others get host_mask[e] = 1 and expert_slot[e] = -1, take no
 * slot and are not inserted (their FFN is the host's to run; host execution is
 * not part of this library).  *n_fills = q*; stats count all m misses and
 * q* * entry_bytes of fills.  pcie_mbps, host_mbps: measured bandwidths in
 * MB/s, >= 0, not both 0 (host_mbps = 0 gives cache_lookup_update).
 * host_mask: device array of E bytes.  Capacity and id errors as in
 * cache_lookup_update (on error only status and *n_fills = 0 are written). */
int cache_lookup_update_split(const moe_cache_t* cache, int layer, const int32_t* topk_ids, int T,
                              int k, int pcie_mbps, int host_mbps, int32_t* expert_slot,
                              moe_fill_t* fills, int32_t* n_fills, uint8_t* host_mask,
                              hipStream_t stream);

/* Copy the n_fills missed entries from the pinned host pool into their slots
 * over PCIe (benchmark page, runtime-tier table: the PCIe link moves selected
 * experts into the GPU cache).  fills_host: host copy of the records written
 * by cache_lookup_update.  Issues hipMemcpyAsync host-to-device on
 * copy_stream, merging records whose slots and pool entries are both
 * consecutive.  Returns MOE_ERANGE (nothing enqueued) for a record outside
 * [0, S) x [0, L) x [0, E) or past the pool (layer*E + expert >= pool_entries).
 * Not capture-safe (the count is host data). */
int cache_fill(const moe_cache_t* cache, const moe_fill_t* fills_host, int n_fills,
               hipStream_t copy_stream);

/* Device-driven miss fills, the graph-capturable form of cache_fill (benchmark
 * page, feature cards: routing-dependent control data stays on the device so
 * execution stays graph-compatible; runtime-tier table: the PCIe link moves
 * selected experts into the GPU cache).  Reads *n_fills and fills[0 .. *n_fills)
 * from device memory, as cache_lookup_update wrote them, and copies each entry
 * (layer, expert) of cache->host_pool into arena slot `slot` with a kernel that
 * reads the pool over PCIe.  The launch shape does not depend on the count, so
 * lookup -> cache_fill_device -> FFN can be captured in one graph with no host
 * synchronisation.
 *   cache->host_pool: pinned host memory mapped for device access at its host
 *   address (hipHostMalloc, or torch pin_memory); 16-byte aligned, as are the
 *   arena and entry_bytes.
 *   fills, n_fills: device memory; max_fills: capacity of fills (host int).
 * Device errors (sticky, in cache->status): *n_fills outside [0, max_fills]
 * sets MOE_ERANGE and copies nothing; a record outside [0, S) x [0, L) x [0, E)
 * or past the pool (layer*E + expert >= pool_entries) sets MOE_ERANGE and is
 * skipped (the others are copied), so no read leaves the pool.  max_fills = 0
 * is a no-op.  Enqueued on `stream`; capture-safe. */
int cache_fill_device(const moe_cache_t* cache, const moe_fill_t* fills, const int32_t* n_fills,
                      int max_fills, hipStream_t stream);

/* Hit and miss masks of the last lookup, so the FFN of resident experts can run
 * while the misses are being copied in (RTX-4090 page, "How the MoE memory
 * hierarchy works": hits run from VRAM; benchmark page, runtime-tier table:
 * misses move over PCIe).  With n = *n_fills:
 *   miss_mask[e] = 1 if expert_slot[e] >= 0 and some fills[i < n].expert == e,
 *   hit_mask[e]  = 1 if expert_slot[e] >= 0 and no record names e, else 0.
 * expert_slot, fills, n_fills as written by cache_lookup_update; masks are
 * device arrays of E bytes, usable as moe_expert_ffn's expert_mask.  Hits and
 * misses use disjoint slots, so moe_expert_ffn(hit_mask) may run concurrently
 * with cache_fill / cache_fill_device, and moe_expert_ffn(miss_mask) after the
 * fill.  Device errors (status nullable, sticky): n outside [0, E] (masks all 0)
 * or a record's expert outside [0, E) set MOE_ERANGE.  1 <= E <= 1024.
 * Capture-safe. */
int cache_fill_masks(const int32_t* expert_slot, const moe_fill_t* fills, const int32_t* n_fills,
                     int E, uint8_t* hit_mask, uint8_t* miss_mask, int32_t* status,
                     hipStream_t stream);

/* Elastic resize of the expert cache at a safe point (benchmark page, "elastic
 * cache" feature card: GPU expert capacity can be reconfigured at a safe runtime
 * point without reloading the host-resident pool).  new_cache has its own S'
 * slots, tables and arena (same L, E, entry_bytes; arenas must not overlap;
 * 1 <= S' <= 4096); host_pool is not touched.  The new tables are rebuilt from
 * the old ones: the min(S', resident) entries used most recently (stamp
 * descending, ties to the lower old slot) are kept, placed in new slots 0..n-1
 * in ascending order of their old slot, with their stamps; their arena entries
 * are copied device to device; the other new slots are empty; clock and stats
 * carry over; new status = 0.  The old cache is only read (its memory may be
 * released once the stream has passed this call).  Nothing else may use either
 * cache until the call completes on `stream`.  Capture-safe. */
int cache_resize(const moe_cache_t* old_cache, const moe_cache_t* new_cache, hipStream_t stream);

/* Full-layer streaming for prefill (llama page, "Official project overview";
 * benchmark page, "How FreeToken serves large MoE models"): waits on
 * wait_before (nullable; the event that marks the end of the last compute
 * reading dst), then copies `bytes` from host_src (pinned) to dst (device) in
 * n_chunks hipMemcpyAsync calls on copy_stream, then records `done`
 * (nullable).  Capture-safe. */
int layer_stream_prefetch(const void* host_src, void* dst, size_t bytes, int n_chunks,
                          hipStream_t copy_stream, hipEvent_t wait_before, hipEvent_t done);

/* ---- measurement helpers ---------------------------------------------------- */

/* Streams `bytes` (multiple of 16) from src and writes one word per
 * workgroup to sink[0 .. 4096) (achievable HBM read bandwidth probe). */
int moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Plain device copy of `bytes` (multiple of 16): reference kernel of known
 * traffic for scaling hardware byte counters. */
int moe_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CACHE_H */
