/*
 * mc.h — C ABI of the MI355X (gfx950) routed-MoE layer over a cross-layer LRU
 * expert slot cache ("mc" = MoE cache).
 *
 * The operations follow the FreeToken pages:
 *   [jjl357] "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
 *            Execution" (jjl357.github.io blog)
 *   [qiita]  "FreeTokenってなんだ？ ─ 8GBノートPCで35Bを動かす判断基準" (Qiita)
 *   [wanger] "FreeToken hybrid MoE 后端：带宽比如何决定专家「搬」还是「算」"
 *   [juhe]   juhe.plus explainer of FreeToken on an 8 GB RTX 4060 Laptop
 *
 * Conventions for every call
 *   - Ownership: the caller allocates and frees every buffer (device memory,
 *     pinned host memory).  The library never frees caller memory.  No hot-path
 *     call allocates device memory; the exceptions are the set-up calls that say
 *     so (mc_bandwidth_profile: a small fill list of its own, freed before it
 *     returns; mc_hybrid_stage_alloc: pinned host staging).  The only
 *     library-owned long-lived object is mc_host_pool (CPU worker threads).
 *   - Asynchrony: calls enqueue work on the given HIP stream and return; results
 *     are visible to the host after the stream is synchronised.  Counts written
 *     by the device (n_fill, n_host, ...) are device int32s.
 *   - Valid counts: where a call takes `const int32_t* n_tok`, NULL means all T
 *     rows are valid; otherwise it is a DEVICE pointer to the number of valid
 *     rows (0 <= *n_tok <= T), read by the kernels, so a fixed-shape call can be
 *     captured once in a hipGraph and replayed for any batch size up to T
 *     ([jjl357] "8.2 把控制流表示成数据": fixed-size buffers plus device-resident
 *     valid counts).
 *   - Errors: arguments are validated on the host before anything is enqueued;
 *     a bad argument returns MC_EINVAL, a failing HIP call MC_EHIP, with a
 *     message from mc_last_error().  Bad device data (an expert id outside
 *     [-1, E), a slot outside [-1, S)) is never dereferenced: the route is
 *     treated as absent and the cache's stats[MC_STAT_ERR] counter is raised.
 *     No call exits the process or lets an exception cross the ABI.
 *   - Threading: calls are reentrant; one mc_cache must be used from one stream
 *     at a time (calls on one cache are ordered by that stream).
 */
#ifndef MC_H
#define MC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MC_ABI_VERSION 1

typedef enum {
  MC_OK = 0,
  MC_EINVAL = -1,        /* invalid argument (nothing was enqueued)           */
  MC_ENOMEM = -2,        /* a caller-provided workspace/staging is too small  */
  MC_EHIP = -3,          /* a HIP runtime call failed                         */
  MC_EUNSUPPORTED = -4,  /* shape or format the library does not handle      */
  MC_EDEVICE = -5        /* device-side error counter was found non-zero      */
} mc_status;

typedef enum { MC_BF16 = 0, MC_MXFP4 = 1 } mc_wfmt;

/*
 * One set of expert banks: n experts, indexed by slot (device pool) or by flat id
 * l*E + e (host pool).  A flat id / slot indexes the same entry of every bank, so
 * one entry across all banks is one complete expert ([jjl357] "8.4 FTW 权重布局").
 *   MC_BF16 : gate_up  bf16 [n][2I][H];   down bf16 [n][H][I];   *_scale unused
 *   MC_MXFP4: gate_up  u8   [n][2I][H/2]  e2m1 codes
 *             gate_up_scale u8 [n][2I][H/32] e8m0
 *             down     u8   [n][H][I/2]   e2m1 codes
 *             down_scale    u8 [n][H][I/32] e8m0
 * gate_up rows [0, I) are the gate projection, rows [I, 2I) the up projection;
 * byte j of a code row holds element 2j in its low nibble and 2j+1 in its high
 * nibble; one e8m0 scale per 32 consecutive elements along the contraction axis
 * (OCP MX: value = 2^(X-127) * e2m1).  Pointers are device pointers for a device
 * pool, pinned host pointers for a host pool.  Bank bases must be 16-byte aligned.
 */
typedef struct {
  int32_t fmt;            /* mc_wfmt */
  int32_t H, I;           /* hidden size, expert intermediate size */
  int32_t reserved;
  int64_t n;              /* number of experts (slots or flat ids) */
  void *gate_up, *gate_up_scale;
  void *down, *down_scale;
} mc_banks;

/*
 * Cross-layer LRU state, all device memory owned by the caller
 * ([juhe] "生成阶段": slot_for_id / id_of_slot / usage; [jjl357] "3. FreeToken Overview":
 * one pool of slots shared by every layer, a slot = one whole (layer, expert)).
 */
typedef struct {
  int32_t L, E, S;        /* layers, experts per layer, slots */
  int32_t reserved;
  int32_t *slot_of;       /* [L*E]  slot holding flat id, -1 = not resident */
  int32_t *id_of;         /* [S]    flat id held by slot, -1 = empty         */
  int64_t *stamp;         /* [S]    clock of last access, 0 = never used     */
  int64_t *clock;         /* [1]    +1 per lookup call                       */
  int64_t *stats;         /* [8]    see MC_STAT_*                            */
} mc_cache;

enum { MC_STAT_HITS = 0, MC_STAT_MISSES = 1, MC_STAT_FILLS = 2, MC_STAT_HOST = 3,
       MC_STAT_EVICT = 4, MC_STAT_CALLS = 5, MC_STAT_ERR = 6 };

/* ------------------------------------------------------------------------- */
/* Library                                                                   */
/* ------------------------------------------------------------------------- */

int mc_abi_version(void);
/* Message of the last failing call on this thread ("" if none). */
const char* mc_last_error(void);

/*
 * Empty cache: slot_of = -1, id_of = -1, stamp = 0, clock = 0, stats = 0 (enqueued
 * as fill kernels on s, so it may be captured).
 */
int mc_cache_reset(const mc_cache* c, hipStream_t s);

/*
 * Q16 fetched fraction of the misses ([jjl357] "6.5 q* 的推导"; [wanger] "实测版本").
 * If p_ov > 0, f = p_ov / (p_ov + c_ov) from bandwidths measured while the host
 * branch and the link run concurrently; otherwise f = b_p / b_h, and f = 1 when
 * b_h <= b_p (no residual host bandwidth, [jjl357] "6.4").  Returns
 * floor(f * 65536 + 1/2) clamped to [1, 65536]; 0 when there is no usable
 * measurement (p_ov <= 0 and b_p <= 0) — the fixed-cap mode of
 * slot_cache_lookup_evict ([wanger] "1. 启动时": no profile -> fixed fetch cap).
 */
uint32_t mc_fetch_fraction_q16(double b_p, double b_h, double p_ov, double c_ov);

/* ------------------------------------------------------------------------- */
/* Hot path                                                                  */
/* ------------------------------------------------------------------------- */

/*
 * Top-k routing ([jjl357] "1.1 Dense LLM 与 MoE LLM 的区别").
 *   logits   device fp32 [T][E]
 *   topk_ids device int32 [T][k] out: experts by logit descending, equal logits
 *            to the lower id (comparisons on the raw fp32 values)
 *   topk_w   device fp32 [T][k] out: renorm=1: softmax over the k selected
 *            logits; renorm=0: the selected experts' softmax probabilities over
 *            all E logits.
 * 1 <= k <= min(E, 32), 1 <= E <= 1024.  T = 0 enqueues nothing.
 */
int moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
              int32_t* topk_ids, float* topk_w, hipStream_t s);

/*
 * One layer call of the cross-layer LRU ([jjl357] "6.1", "6.7", "8.2";
 * [wanger] "3. ensure_experts_hybrid 内核").  One kernel, one workgroup:
 *   1. clock += 1; U = sorted unique flat ids layer*E + e of the valid routes
 *      (rows t < *n_tok; id -1 = masked route; ids outside [-1, E) count in
 *      stats[ERR] and are ignored).
 *   2. hits: resident members of U, stamped with the clock.  Misses M (ascending),
 *      m = |M|.
 *   3. q: frac_q16 = 0 -> min(m, fixed_cap); otherwise, with f = frac_q16 / 65536,
 *      q is the integer F next to m*f that makes the slower of the two miss branches,
 *      max(F*(1-f), (m-F)*f), smallest, ties to the smaller F ([wanger] "3."); it
 *      equals ceil(f*(m+1)) - 1 <= m.  min_fill != 0 and m >= 1 -> q >= 1.  Then q is
 *      capped by the slots not hit in this call and by kcap.
 *   4. victims: the q slots not hit in this call with the smallest (stamp, slot).
 *      The first q misses are paired in order with the victims: the old
 *      occupant (if any) is evicted, the miss is installed and stamped.
 *   5. the remaining m - q misses are host-computed: no insert, no stamp.
 *   6. slots[t][j] = slot of the route's expert, or -1 (host-computed, masked,
 *      invalid, or t >= *n_tok).
 *   ids       device int32 [T][k] expert-in-layer ids
 *   fill_flat, fill_slot  device int32 [kcap] out: (flat id, slot) of each fill
 *   n_fill    device int32 [1] out: q
 *   host_flat device int32 [kcap] out: flat ids of the host-computed misses, ascending
 *   n_host    device int32 [1] out: m - q
 * frac_q16 in [0, 65536] (65536 = fetch every miss), fixed_cap >= 0,
 * kcap >= T*k, 0 <= layer < L, T*k <= 4096.
 */
int slot_cache_lookup_evict(const mc_cache* c, int32_t layer, const int32_t* ids, int32_t T,
                            int32_t k, const int32_t* n_tok, uint32_t frac_q16, int32_t fixed_cap,
                            int32_t min_fill, int32_t* slots, int32_t* fill_flat,
                            int32_t* fill_slot, int32_t* n_fill, int32_t* host_flat,
                            int32_t* n_host, int32_t kcap, hipStream_t s);

/*
 * Routing and lookup of one decode layer call in a single launch: exactly
 * moe_route(logits, T, c->E, k, renorm, topk_ids, topk_w) followed by
 * slot_cache_lookup_evict(c, layer, topk_ids, T, k, n_tok, ...) with the same
 * outputs, but the ids stay on chip between the two steps ([jjl357] "8.2": the
 * control flow of a step lives in device data, and fewer launches per layer).
 * Argument meaning, layout and limits are those of the two calls (c->E <= 1024).
 */
int moe_route_lookup(const float* logits, int32_t renorm, int32_t* topk_ids, float* topk_w,
                     const mc_cache* c, int32_t layer, int32_t T, int32_t k, const int32_t* n_tok,
                     uint32_t frac_q16, int32_t fixed_cap, int32_t min_fill, int32_t* slots,
                     int32_t* fill_flat, int32_t* fill_slot, int32_t* n_fill, int32_t* host_flat,
                     int32_t* n_host, int32_t kcap, hipStream_t s);

/*
 * Placement without a lookup: flat id flat[i] becomes resident in slot i, for i < n
 * (device list).  For a fixed placement chosen ahead of decode — the static and
 * prefill-time placements the pages compare LRU against ([jjl357] "11.2 Expert Cache
 * Locality"; [qiita] "5. デコード側の答え その1") — and for adopting experts whose bytes
 * are already in the slots.  Only the tables change (bytes: mc_fill_slots); the call
 * advances the clock by one and stamps the installed slots with it, so they are more
 * recent than the empty slots and less recent than anything a later call touches.  The cache must hold no expert in slots [0, n) (right after
 * mc_cache_reset); id -1 leaves its slot empty; other ids outside [0, L*E), duplicates
 * and occupied slots are skipped and counted in stats[MC_STAT_ERR].  A lookup with fixed_cap = 0, min_fill = 0 and
 * frac_q16 = 0 then never fills or evicts, which keeps such a placement fixed.
 */
int mc_cache_install(const mc_cache* c, const int32_t* flat, int32_t n, hipStream_t s);

/*
 * Fill fetch ([jjl357] "6.7" step 3 and "6.8": one fused batch copy of the chosen
 * misses into their victim slots).  Copies every bank of host entry fill_flat[i]
 * into pool entry fill_slot[i] for i < *n_fill, as a kernel that reads the pinned
 * host banks over the host link (no host synchronisation, capturable).
 *   host  pinned host banks indexed by flat id (host->n = L*E), same fmt/H/I as pool
 *   pool  device slot banks (pool->n = S)
 *   fill_flat, fill_slot, n_fill: as written by slot_cache_lookup_evict (device)
 * Entries with a flat id outside [0, host->n) or a slot outside [0, pool->n) are
 * skipped.  kcap = capacity of the lists, 0..65535 (MC_EINVAL otherwise).
 */
int mc_fill_slots(const mc_banks* host, const mc_banks* pool, const int32_t* fill_flat,
                  const int32_t* fill_slot, const int32_t* n_fill, int32_t kcap, hipStream_t s);

/*
 * Forget the device translations the library remembers for pinned host memory in
 * [p, p + bytes) (bytes = 0: the one address p); returns how many were dropped.
 * Calls made outside stream capture always check their host banks with the runtime;
 * a call made while its stream is being captured uses the translation remembered
 * from an earlier call on the same address.  A caller that frees pinned banks and may
 * capture again calls this first, so a later capture cannot take a stale translation
 * (mc_hybrid_stage_free does it for the stage).  p = NULL is MC_EINVAL.
 */
int mc_host_forget(const void* p, size_t bytes);

/* Bank bits of mc_fill_slots_banks. */
enum { MC_BANK_GATE_UP = 1, MC_BANK_GATE_UP_SCALE = 2, MC_BANK_DOWN = 4, MC_BANK_DOWN_SCALE = 8,
       MC_BANK_ALL = 15 };

/*
 * mc_fill_slots restricted to the banks in `banks` (a nonzero mask of MC_BANK_*): the
 * other banks of the slots are left as they are.  Used with a gate_up-only
 * fill-through pass (mc_fill_list.mode = MC_FILL_GATE_UP), which writes the gate_up
 * banks while this copies the down banks on another stream.
 */
int mc_fill_slots_banks(const mc_banks* host, const mc_banks* pool, const int32_t* fill_flat,
                        const int32_t* fill_slot, const int32_t* n_fill, int32_t kcap,
                        uint32_t banks, hipStream_t s);

/*
 * Fill list of one lookup call, handed to moe_experts_decode so that the fill of the
 * chosen misses happens inside the expert pass ("fill-through"): a route whose slot
 * is fill_slot[i] (i < *n_fill) reads its weights from host entry fill_flat[i] over
 * the host link, and the same pass writes every byte of that entry into the slot.
 * The slot then holds exactly what mc_fill_slots would have copied; the host link
 * carries each filled expert once, and the hits' HBM traffic runs beside it instead
 * of after it.  All list pointers are device memory, as written by
 * slot_cache_lookup_evict; host = pinned host banks by flat id (same fmt/H/I as the
 * pool).  Entries with a flat id outside [0, host->n) are ignored (the route then
 * reads its slot as usual).
 */
enum { MC_FILL_THROUGH = 0, MC_FILL_GATE_UP = 1, MC_FILL_WITH_GATE_UP = 2 };

typedef struct {
  const mc_banks* host;
  const int32_t* fill_flat;  /* [kcap] */
  const int32_t* fill_slot;  /* [kcap] */
  const int32_t* n_fill;     /* [1]    */
  int32_t kcap;
  /* MC_FILL_THROUGH: both passes read the host and fill through.
   * MC_FILL_GATE_UP: only the gate_up pass reads the host and writes the gate_up banks;
   *   the down pass reads the slots, whose down banks the caller fills
   *   (mc_fill_slots_banks with MC_BANK_DOWN | MC_BANK_DOWN_SCALE, e.g. on another
   *   stream, concurrently with the gate_up pass).
   * MC_FILL_WITH_GATE_UP: the gate_up pass fills through its banks and its launch also
   *   copies the down banks of every listed entry (workgroups of their own beside the
   *   gate_up workgroups), so the down pass reads the slots; one token per call gets the
   *   single launch, several tokens a separate copy between the two passes.  The caller
   *   runs no mc_fill_slots. */
  int32_t mode;
  /* NULL, or an event the down pass waits for (the caller's down-bank fill) */
  hipEvent_t down_after;
} mc_fill_list;

/*
 * Workspace bytes of moe_experts_decode for up to T tokens x k routes of experts with
 * hidden size H and intermediate size I.
 */
size_t moe_experts_decode_ws_bytes(int32_t T, int32_t k, int32_t H, int32_t I);

/*
 * Slot-indirected SwiGLU experts and gated combine on the GPU
 * ([jjl357] "1.1", "6.7" step 5; [wanger] "代码全链路": GPU routes of the hybrid
 * split carry gate 0 for host routes).
 *   y_acc[t][:] (+)= sum_j w[t][j] * Expert(pool[slots[t][j]])(x[t])
 *                    (+ Expert(shared[0])(x[t]) with weight 1 if shared != NULL)
 * for t < *n_tok, over routes with slots[t][j] >= 0; each distinct slot's weights
 * are read once for all tokens that route to it ([jjl357] "6.1": dedup).
 * Expert(x) = W_down (silu(W_gate x) * (W_up x)), fp32 accumulation; x bf16 [T][H].
 *   y_acc      fp32 [T][H]: accumulate = 1 adds to it, accumulate = 0 overwrites it
 *              (rows t >= *n_tok are then set to 0).
 *   y_bf16     NULL, or bf16 [T][H] written with bf16_rne(y_acc) (rows t >= *n_tok = 0),
 *              so a layer with no host branch needs no separate rounding pass.
 *   pool       device slot banks; shared: NULL or a device bank whose entry 0 is the
 *              layer's shared expert (same fmt, H, I).
 *   ws         device workspace of moe_experts_decode_ws_bytes(T, k, H, I) bytes (the
 *              gate_up results h, each route's gated partial output and the down pass's
 *              arrival counters), 16-byte aligned; one workspace per call in flight (two
 *              calls that overlap on one workspace race).
 *   fill       NULL (every routed slot is resident), or the fill list of this call's
 *              lookup (mc_fill_list): those slots are read from the host and written
 *              in the same pass, so no separate mc_fill_slots is needed.
 * Two kernel launches: gate_up + SwiGLU, then down.  One token (T = 1): dot-product
 * kernels over whole row slices, the down rows of every route of the token summed in
 * one workgroup per block of rows.  Several tokens: both passes unit-major on the
 * matrix cores (a unit = one distinct slot, or the shared expert); each unit's down rows
 * produce every route's gated partial for a block of rows and the last unit to finish a
 * block adds the partials of each token in route order.  Every order is fixed, so
 * results are run-to-run identical.  Needs H % 64 == 0, I % 64 == 0, T <= 64,
 * T*k <= 1024.
 */
int moe_experts_decode(const void* x_bf16, const int32_t* slots, const float* w, int32_t T,
                       int32_t k, const int32_t* n_tok, const mc_banks* pool,
                       const mc_banks* shared, void* ws, size_t ws_bytes, float* y_acc,
                       int32_t accumulate, void* y_bf16, hipStream_t s, const mc_fill_list* fill);


/*
 * moe_experts_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under hipGraph capture that must not call hipMalloc, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results and
 * kernels as moe_experts_decode; the workspace is a file-scope device array of the
 * library, moe_experts_decode_noalloc_max_bytes() bytes (4 MiB) per GPU, held until the
 * process ends.  Nothing is allocated by the call (no hipMalloc, no allocating library
 * routine); the array's device address is looked up once per GPU on its first call.
 * A call whose moe_experts_decode_ws_bytes(T, k, H, I) exceeds the array returns
 * MC_ENOMEM with a message (nothing is enqueued).  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents (no part of it needs clearing):
 * calls that overlap on one GPU — on two streams, or from two threads — race and must
 * be ordered by the caller.
 */
int moe_experts_decode_noalloc(const void* x_bf16, const int32_t* slots, const float* w, int32_t T,
                               int32_t k, const int32_t* n_tok, const mc_banks* pool,
                               const mc_banks* shared, float* y_acc, int32_t accumulate,
                               void* y_bf16, hipStream_t s, const mc_fill_list* fill);
/* Size of the array moe_experts_decode_noalloc works in (bytes). */
size_t moe_experts_decode_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------- */
/* Prefill                                                                   */
/* ------------------------------------------------------------------------- */

/*
 * Stable grouping of a prefill chunk's routes by expert (the token sort in front of
 * the grouped GEMM; [jjl357] "6.8": grouped GPU execution).  Route r = t*k + j for
 * t < *n_tok (NULL = T) with 0 <= ids[r] < E:
 *   counts  [E]    routes per expert
 *   offsets [E+1]  exclusive prefix sum of counts
 *   perm    [T*k]  perm[offsets[e] .. offsets[e+1]) = the routes of expert e in
 *                  ascending r (the other entries are left untouched)
 * ws: device scratch of at least E*16 + (E+1)*4 bytes.  All device memory.
 * E <= 1024.
 */
int mc_prefill_sort_routes(const int32_t* ids, int32_t T, int32_t k, const int32_t* n_tok,
                           int32_t E, void* ws, size_t ws_bytes, int32_t* counts,
                           int32_t* offsets, int32_t* perm, hipStream_t s);

/*
 * Whole-layer prefetch of the next layer's experts ([jjl357] "4.2 双缓冲时间线":
 * buffer B is filled over the host link while buffer A computes).  On stream `copy`:
 * wait for dst_free (may be NULL), copy host entries [first_flat, first_flat + E) of
 * every bank into dst entries [0, E) with hipMemcpyAsync (SDMA), record done (may be
 * NULL).  The caller makes the compute stream wait on `done` before using dst and
 * records dst_free after the last kernel that reads dst's previous contents.
 */
typedef struct {
  const mc_banks* host_src;  /* pinned host banks by flat id */
  int64_t first_flat;        /* flat id of expert 0 of the next layer (= layer * E) */
  const mc_banks* dst;       /* device layer buffer, >= E entries */
  hipStream_t copy;
  hipEvent_t dst_free;
  hipEvent_t done;
} mc_prefetch;

size_t moe_experts_prefill_ws_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I);

/*
 * Prefill MoE layer over a resident layer buffer (entry e = expert e of the layer):
 *   y[t] = bf16_rne( sum_j w[t][j] * Expert_{ids[t][j]}(x[t]) )   for t < *n_tok (else 0)
 * computed as a stable token sort by expert, a grouped gate_up GEMM with the SwiGLU
 * epilogue (bf16 MFMA; MXFP4 -> bf16 is exact), a grouped down GEMM (fp16 MFMA on fp16
 * h and MXFP4 -> fp16 weights), fp32 accumulation, and a fixed-order sum of each token's
 * k gated route outputs.  W_down is consumed exactly: a row whose block exponents X-127
 * leave fp16's exact range [-23, 13] is dequantised at a power-of-two offset that the
 * epilogue undoes (blocks more than 36 binades below the row's largest then round, a
 * share of the output below the fp32 accumulation's own rounding).  h is held in fp16:
 * a value beyond +-65504 becomes +-inf and is recorded in the workspace's status word
 * (moe_experts_prefill_status); values below fp16's normal range keep an absolute
 * error under 2^-25.
 * If next != NULL the next layer's prefetch (see mc_prefetch) is enqueued first on
 * its own stream, so it overlaps this layer's compute.
 *   x bf16 [T][H], ids int32 [T][k] (expert-in-layer; invalid ids contribute nothing),
 *   w fp32 [T][k], y bf16 [T][H]; ws of moe_experts_prefill_ws_bytes(T, k, E, H, I).
 * MXFP4 only; H % 256 == 0, I % 128 == 0, E <= 1024.
 */
int moe_experts_prefill(const void* x_bf16, const int32_t* ids, const float* w, int32_t T,
                        int32_t k, const int32_t* n_tok, int32_t E, const mc_banks* layer_buf,
                        void* ws, size_t ws_bytes, void* y_bf16, hipStream_t s,
                        const mc_prefetch* next);

/*
 * A prefill layer in parts, for a slot pool too small for the whole-layer double buffer
 * ([jjl357] "4.3" last paragraph, "4.4"; [juhe] "Prefill 为什么不能也按需加载": without
 * room for two whole layers the engine falls back to loading the routed experts on
 * demand).  The steps of moe_experts_prefill, run separately on one workspace:
 *   MC_PF_SORT     the stable token sort of ids (also writes each expert's route count
 *                  to the device array counts [E] when counts != NULL);
 *   MC_PF_EXPERTS  the grouped gate_up / SwiGLU / down GEMMs of the experts e with
 *                  entry_of[e] >= 0 (device int32 [E]), whose weights are entry
 *                  entry_of[e] of part_buf; each of their routes' gated outputs is kept
 *                  in the workspace;
 *   MC_PF_COMBINE  y = bf16 of each token's fixed-order sum over its valid routes.
 * A layer is one SORT, EXPERTS steps whose parts together cover every routed expert
 * once, and one COMBINE, in stream order on the same workspace; the result is then
 * bit-identical to moe_experts_prefill's.  Arguments and limits as moe_experts_prefill.
 */
enum { MC_PF_SORT = 1, MC_PF_EXPERTS = 2, MC_PF_COMBINE = 4, MC_PF_ALL = 7 };
int moe_experts_prefill_part(const void* x_bf16, const int32_t* ids, const float* w, int32_t T,
                             int32_t k, const int32_t* n_tok, int32_t E, const mc_banks* part_buf,
                             const int32_t* entry_of, int32_t steps, void* ws, size_t ws_bytes,
                             int32_t* counts, void* y_bf16, hipStream_t s);

/*
 * Status of the last moe_experts_prefill call made with workspace ws: waits for stream
 * s, then *status = the call's status bits (1: an h value exceeded the fp16 range).
 * Returns MC_EDEVICE with a message when a bit is set, MC_OK otherwise.  Synchronous.
 */
int moe_experts_prefill_status(const void* ws, hipStream_t s, uint32_t* status);

/* ------------------------------------------------------------------------- */
/* Hybrid split / merge and the host branch                                  */
/* ------------------------------------------------------------------------- */

/* Persistent CPU worker pool ([jjl357] "8.3": persistent C++ workers pinned to cores). */
typedef struct mc_host_pool mc_host_pool;
/* n_threads >= 1 compute threads: one dispatcher thread, which serves the hybrid stages
 * registered with the pool (see hybrid_split_merge; it polls while calls keep coming)
 * and computes, plus n_threads - 1 workers.  cpu_ids: NULL pins thread i to a distinct
 * physical core of the CPUs this process may use (one hardware thread per core, in
 * (package, core) order, further hardware threads only when there are more threads than
 * cores), leaving the first core of that order to the rest of the process (the thread
 * that launches GPU work); threads beyond the remaining CPUs stay unpinned.  Else
 * n_threads CPU ids, thread 0 being the dispatcher, -1 leaving a thread unpinned.  NULL
 * on failure. */
mc_host_pool* mc_host_pool_create(int32_t n_threads, const int32_t* cpu_ids);
/* The CPU of each pool thread (-1 = not pinned): writes min(n, n_threads) entries and
 * returns n_threads (MC_EINVAL for a NULL pool). */
int32_t mc_host_pool_cpus(const mc_host_pool* p, int32_t* cpus, int32_t n);
void mc_host_pool_destroy(mc_host_pool* p);

/*
 * Host expert FFN, synchronous (used by the hybrid branch and by tests):
 *   y[t][:] += sum_j w[t][j] * Expert(host[layer*E + flat_ids... ]) — precisely, for
 *   every (t, j) with ids[t][j] >= 0: y[t] += w[t][j] * Expert(host entry
 *   layer*E + ids[t][j])(x[t]).  Dequantisation happens inside the dot products
 *   ([jjl357] "8.3": SIMD kernels dequantise in-kernel).  All pointers are host
 *   memory: x bf16 [T][H], ids int32 [T][k], w fp32 [T][k], y fp32 [T][H].
 *   pool may be NULL (runs on the calling thread).
 */
int mc_host_experts(mc_host_pool* pool, const void* x_bf16, const int32_t* ids, const float* w,
                    int32_t T, int32_t k, int32_t layer, int32_t E, const mc_banks* host,
                    float* y);

/*
 * Start-up bandwidth profile ([wanger] "第一层带宽比：选后端" and "实测版本：overlap 带宽取代
 * 假设").  Measures the two paths a hybrid decode layer runs, on this machine:
 *   pcie_gbs     the fill kernel (mc_fill_slots) copying n host entries into pool slots
 *                [0, n) per call, alone (bytes of the n experts per second)
 *   cpu_gbs      mc_host_experts for one token routed to n host entries per call, alone
 * Successive calls of both paths take the next n entries of a window of
 * W = min(host->n, max(n, ceil(1 GiB / expert bytes))) entries, so they read host DRAM
 * as a decode step does rather than the CPU's last-level cache.
 *   pcie_ov_gbs, cpu_ov_gbs  the same two while both run at once, each sized from its
 *                stand-alone rate to take about seconds/2
 *   frac_q16     mc_fetch_fraction_q16(pcie_gbs, cpu_gbs, pcie_ov_gbs, cpu_ov_gbs)
 *   hybrid       mc_recommend_backend(cpu_gbs, pcie_gbs, threshold)
 * Synchronous (waits on s; not for capture); about `seconds` of wall time.  Overwrites
 * pool slots [0, n) and uses device memory of its own for the fill list.  host: pinned
 * host banks; pool: device banks (same fmt/H/I); workers: NULL = calling thread.
 * 1 <= n_experts <= min(host->n, pool->n, 4096); 0 < seconds <= 60; threshold > 0.
 */
typedef struct {
  double pcie_gbs, cpu_gbs, pcie_ov_gbs, cpu_ov_gbs;
  double expert_bytes;       /* bytes of one expert entry (all banks) */
  uint32_t frac_q16;
  int32_t hybrid;            /* 1 = hybrid, 0 = offload */
} mc_bw_profile;

int mc_bandwidth_profile(const mc_banks* host, const mc_banks* pool, mc_host_pool* workers,
                         int32_t n_experts, double seconds, double threshold, hipStream_t s,
                         mc_bw_profile* out);

/*
 * Backend choice ([wanger] "第一层带宽比：选后端"): 1 (hybrid) iff
 * cpu_gbs > threshold * pcie_gbs, else 0 (offload).  The page's threshold is 2.0.
 */
int32_t mc_recommend_backend(double cpu_gbs, double pcie_gbs, double threshold);

/* Pinned staging bytes of one hybrid layer call (header, request and completion
 * words, x, ids, w, y_host). */
size_t mc_hybrid_stage_bytes(int32_t T, int32_t k, int32_t H);

/*
 * Staging memory of a hybrid layer call ([jjl357] "6.8": the CPU writes its partial to
 * pinned memory).  Fine-grained (coherent) pinned host memory, zeroed, so that the GPU
 * and the host see each other's stores to it while a kernel runs.  Returns NULL on
 * failure (mc_last_error).  mc_hybrid_stage_free synchronises the device, removes the
 * stage from the worker pool's dispatcher and frees it; NULL is a no-op.
 * mc_hybrid_stage_errors: merge waits on the stage that ran out (0 normally).
 */
void* mc_hybrid_stage_alloc(size_t bytes);
int mc_hybrid_stage_free(void* stage);
uint32_t mc_hybrid_stage_errors(const void* stage);

typedef struct {
  const void* x_bf16;        /* device bf16 [T][H]                                   */
  const int32_t* ids_raw;    /* device int32 [T][k]: router ids (expert-in-layer)    */
  const int32_t* slots;      /* device int32 [T][k]: slot_cache_lookup_evict output  */
  const float* w;            /* device fp32 [T][k]: router gates                     */
  int32_t T, k, layer, E;
  const int32_t* n_tok;      /* device valid count or NULL                           */
  const mc_banks* host;      /* pinned host banks by flat id                         */
  mc_host_pool* pool;        /* CPU workers                                          */
  void* pinned_stage;        /* from mc_hybrid_stage_alloc, mc_hybrid_stage_bytes      */
  size_t stage_bytes;
  float* gpu_w;              /* device fp32 [T][k] out: w where slot >= 0, else 0   */
  int32_t* host_ids;         /* device int32 [T][k] out: raw id where slot < 0, else -1 */
  float* y_acc;              /* device fp32 [T][H]: GPU partial (moe_experts_decode) */
  float* y_host;             /* device fp32 [T][H] out: the host partial (rows < n_tok) */
  void* y_bf16;              /* device bf16 [T][H] out: bf16(y_acc + y_host)         */
} mc_hybrid;

enum { MC_SPLIT_SUBMIT = 0, MC_MERGE = 1 };

/*
 * Exact split and merge of one decode layer ([jjl357] "6.2", "6.8", "6.9";
 * [wanger] "代码全链路"; [juhe] "为什么可以直接相加").
 * MC_SPLIT_SUBMIT: one kernel writes gpu_w and host_ids (complementary masks: every
 *   valid route is on exactly one side), writes x / host ids / w / the valid count /
 *   the layer into the stage and then raises the stage's request number (a call with
 *   no host route leaves the stage alone and its merge does not wait).  The worker
 *   pool's dispatcher thread (polling the stages it serves) computes the host partial
 *   into the stage and raises the completion number; meanwhile the GPU continues
 *   with fills and moe_experts_decode.  No host function and no copy is enqueued, so
 *   the sequence can be captured in a hipGraph and replayed.
 * MC_MERGE: one kernel waits for the completion number (bounded, about 4 s: a wait
 *   that runs out is counted, see mc_hybrid_stage_errors, and leaves wrong values),
 *   writes the host partial to y_host and y_bf16 = bf16_rne(y_acc + y_host) — one
 *   rounding.
 * Every SPLIT_SUBMIT must be followed by a MERGE on the same stream before the stage
 * is reused.  A stage keeps the (T, k, H, E, host banks, worker pool) of its first
 * call (another set is MC_EINVAL).  The pool must outlive the calls on its stages.
 */
int hybrid_split_merge(const mc_hybrid* h, int32_t phase, hipStream_t s);

/*
 * Final bf16 output of a layer with no host branch: y_bf16 = bf16_rne(y_acc) for
 * rows t < *n_tok (rows beyond are set to 0).
 */
int mc_finish_bf16(const float* y_acc, int32_t T, int32_t H, const int32_t* n_tok, void* y_bf16,
                   hipStream_t s);

#ifdef __cplusplus
}
#endif
#endif /* MC_H */
