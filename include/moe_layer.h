/*
 * moe_layer.h -- C ABI of the routed mixture-of-experts verify layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is one routed-MoE FFN block of a Step-3.5/3.7-Flash or Step-5
 * transformer applied to a small decode/verify batch: the last accepted
 * token plus up to three MTP drafts ("Support Step3.5/3.7 flash mtp3",
 * Overview, data-flow trace: the 4-token target batch with all logits on),
 * or to a prefill micro-batch of 512 tokens ("Step-5 Preview GGUF", Run the
 * server, -ub 512; Validation and measured performance, microbatch 512).
 * Step-5 uses hidden size 4096 and 352 routed experts with 8 selected per
 * token ("Step-5 Preview GGUF", Model background, configuration table).
 * Routers are F32, shared experts Q8_0 and routed experts Q4_K in the mixed
 * recipes ("Step-5 Preview GGUF", Precision distribution table; "Step 3.7
 * Flash Mixed-Quant GGUF", Tensor recipe); the 2-bit Step-5 recipes store
 * routed matrices in Q2_K and Q3_K, Q2_K-Protected2 with Q2_K gate/up and
 * Q3_K down ("Step-5 Preview GGUF", Tensor-type table); every recipe stores
 * the MTP heads' matrices in Q6_K (same table).
 *
 * What one call computes, for each token t of x [M][H]:
 *   l[e]    = sum_h router[e][h] * x[t][h]                      (F32 router)
 *   ids[j]  = the top_k experts by descending l, ties to the lower index
 *   w[j]    = exp(l[ids[j]] - l_max) / sum_i exp(l[ids[i]] - l_max)
 *             (softmax over all experts restricted to the selection and
 *              renormalised; the two are equal in exact arithmetic)
 *   o_j     = Wd_e (silu(Wg_e x_t) * (Wu_e x_t)),  e = ids[j],  silu(g) = g/(1+e^-g)
 *   s       = the same SwiGLU FFN with the shared expert (absent if shared_ffn == 0)
 *   y[t]    = s + sum_{j=0..top_k-1} w[j] * o_j        (summed in slot order)
 * The pages name the router's precision and the tensor types but not the
 * router formula, the activation or any byte layout; the formula above and
 * the layouts below are this library's contract.
 *
 * BYTE LAYOUTS (planar block quantisation; all little-endian)
 *   MOE_F32  [rows][cols] float.
 *   MOE_Q8_0 rows x cols, cols % 32 == 0, nb = cols / 32.  Blocks of 32
 *            weights with one fp16 scale d and 32 int8 quants q, w = d * q.
 *            Bytes [0, 2*rows*nb): fp16 d of block (r, b) at 2*(r*nb + b).
 *            Bytes from Q = round_up(2*rows*nb, 256): int8 q of weight
 *            (r, c) at Q + r*cols + c.  Total Q + rows*cols bytes.
 *   MOE_Q4_K rows x cols, cols % 256 == 0, ns = cols / 256.  Super-blocks
 *            of 256 weights: fp16 d and dmin, 8 sub-blocks of 32 weights
 *            with a 6-bit scale sc and a 6-bit min m, 4-bit quants q,
 *            w = d*sc_s*q - dmin*m_s.
 *            Bytes [0, 16*rows*ns): 16-byte header of super-block (r, b) at
 *            16*(r*ns + b): fp16 d, fp16 dmin, then 12 bytes holding a 96-bit
 *            little-endian stream with sc_s in bits [6s, 6s+6) and m_s in
 *            bits [48+6s, 54+6s).
 *            Bytes from 16*rows*ns: 128 quant bytes of super-block (r, b) at
 *            16*rows*ns + 128*(r*ns + b); sub-block s in bytes [16s, 16s+16)
 *            of them; weight i of a sub-block in byte i/2, low nibble for
 *            even i, high nibble for odd i.  Total 144*rows*ns bytes.
 *   MOE_Q2_K rows x cols, cols % 256 == 0, ns = cols / 256, routed experts
 *            only.  Super-blocks of 256 weights: fp16 d and dmin, 16
 *            sub-blocks of 16 weights with a 4-bit scale sc and a 4-bit min
 *            m, 2-bit quants q, w = d*sc_s*q - dmin*m_s.
 *            Bytes [0, 4*rows*ns): fp16 d then fp16 dmin of super-block
 *            (r, b) at 4*(r*ns + b).
 *            Bytes from S = round_up(4*rows*ns, 256): 16 scale bytes of
 *            super-block (r, b) at S + 16*(r*ns + b), byte s = sc_s | m_s << 4.
 *            Bytes from Q = round_up(S + 16*rows*ns, 256): 64 quant bytes of
 *            super-block (r, b) at Q + 64*(r*ns + b); sub-block s in bytes
 *            [4s, 4s+4) of them; weight i of a sub-block in byte i % 4, bits
 *            [2*(i/4), 2*(i/4)+2).  Total Q + 64*rows*ns bytes.
 *   MOE_Q3_K rows x cols, cols % 256 == 0, ns = cols / 256, routed experts
 *            only.  Super-blocks of 256 weights: fp16 d, 16 sub-blocks of 16
 *            weights with a 6-bit scale S, 3-bit quants Q,
 *            w = d*(S_s - 32)*(Q - 4).
 *            Bytes [0, 2*rows*ns): fp16 d of super-block (r, b) at
 *            2*(r*ns + b).
 *            Bytes from S = round_up(2*rows*ns, 256): 16 scale bytes of
 *            super-block (r, b) at S + 16*(r*ns + b), byte s = S_s (bits
 *            6..7 zero).
 *            Bytes from L = round_up(S + 16*rows*ns, 256): the low two bits
 *            of every Q, 64 bytes per super-block at L + 64*(r*ns + b), laid
 *            out as the Q2_K quants.
 *            Bytes from G = round_up(L + 64*rows*ns, 256): the high bit of
 *            every Q, 32 bytes per super-block at G + 32*(r*ns + b); weight i
 *            of sub-block s in byte 4*(s/2) + i % 4, bit 4*(s % 2) + i/4.
 *            Total G + 32*rows*ns bytes.
 *   MOE_Q6_K rows x cols, cols % 256 == 0, ns = cols / 256, routed experts
 *            only.  Super-blocks of 256 weights: fp16 d, 16 sub-blocks of 16
 *            weights with a signed 8-bit scale sc, 6-bit quants Q,
 *            w = d*sc_s*(Q - 32).
 *            Bytes [0, 2*rows*ns): fp16 d of super-block (r, b) at
 *            2*(r*ns + b).
 *            Bytes from S = round_up(2*rows*ns, 256): 16 int8 scales of
 *            super-block (r, b) at S + 16*(r*ns + b).
 *            Bytes from L = round_up(S + 16*rows*ns, 256): the low four bits
 *            of every Q, 128 bytes per super-block at L + 128*(r*ns + b),
 *            laid out as the Q4_K quants (32-weight group g in bytes
 *            [16g, 16g+16), weight i of it in byte i/2, low nibble for even
 *            i); sub-block s is group s/2, weights 16*(s%2) onward.
 *            Bytes from G = round_up(L + 128*rows*ns, 256): the high two
 *            bits of every Q, 64 bytes per super-block at G + 64*(r*ns + b);
 *            weight i of group g at byte 8g + 4*(i/16) + (i%8)/2, bits
 *            4*((i/8)%2) + 2*(i%2) and the next one.
 *            Total G + 64*rows*ns bytes.
 *   Expert tensors are stacked experts-outermost and stored as one tensor:
 *   gate and up are (E*F) x H, down is (E*H) x F; expert e owns rows
 *   [e*F, (e+1)*F) (resp. [e*H, (e+1)*H)).  The shared expert's gate and up
 *   are Fs x H, its down H x Fs.  Rows run along the input dimension.
 *
 * OWNERSHIP AND ORDERING
 *   Every pointer argument except desc/weights structs and the event array
 *   is a DEVICE pointer owned by the caller.  The library allocates no
 *   memory and keeps no state between calls; calls are re-entrant given
 *   distinct workspaces.  All work is enqueued on hip_stream (a hipStream_t;
 *   NULL = the null stream) and the call returns without synchronising.
 *   Inputs are read-only; outputs must not alias inputs or each other.
 *   Device faults surface at the caller's next synchronisation.
 *
 * ERRORS
 *   Every entry point returns a status (below) and enqueues nothing unless
 *   it returns MOE_OK, except MOE_ERR_LAUNCH, which reports a failure seen
 *   after enqueueing (hipGetLastError).  Shapes are checked before launch:
 *   1 <= n_experts <= 1024; 1 <= top_k <= min(n_experts, 64); hidden,
 *   ffn and shared_ffn multiples of 32 (Q8_0) or 256 (Q4_K, Q2_K, Q3_K,
 *   Q6_K) for the tensors that use them, and a row of at most 512 blocks of
 *   16 bytes (Q8_0: 8192 columns, Q4_K and Q6_K: 16384, Q2_K and Q3_K:
 *   32768); n_tokens >= 0 (0 enqueues nothing).  MOE_Q2_K, MOE_Q3_K or
 *   MOE_Q6_K as shared_type is MOE_ERR_DTYPE.
 */
#ifndef SVR_MOE_LAYER_H
#define SVR_MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tensor types. */
#define MOE_F32 0
#define MOE_Q8_0 1
#define MOE_Q4_K 2
#define MOE_Q2_K 3
#define MOE_Q3_K 4
#define MOE_Q6_K 5

/* Status codes. */
#define MOE_OK 0
#define MOE_ERR_NULL 1       /* a required pointer is NULL or a size negative */
#define MOE_ERR_SHAPE 2      /* unsupported shape */
#define MOE_ERR_DTYPE 3      /* unsupported tensor type */
#define MOE_ERR_WORKSPACE 4  /* workspace smaller than moe_workspace_bytes() */
#define MOE_ERR_LAUNCH 5     /* a kernel launch failed */
#define MOE_ERR_ARG 6        /* other invalid argument (e.g. event count) */

/* Layer shape and tensor types. */
typedef struct moe_layer_desc {
  int32_t hidden;      /* H */
  int32_t n_experts;   /* E */
  int32_t top_k;       /* k */
  int32_t ffn;         /* F, routed expert FFN width */
  int32_t shared_ffn;  /* Fs, shared expert FFN width; 0 = no shared expert */
  int32_t expert_type; /* MOE_Q8_0, MOE_Q4_K, MOE_Q2_K, MOE_Q3_K or MOE_Q6_K:
                          routed gate/up, and down unless down_type says
                          otherwise */
  int32_t shared_type; /* MOE_Q8_0 or MOE_Q4_K: shared gate/up/down */
  int32_t flags;       /* reserved: must be 0 (other values: MOE_ERR_ARG) */
  int32_t down_type;   /* routed down: 0 = expert_type, else one of the types
                          expert_type takes */
} moe_layer_desc;

/* Device pointers to the layer's tensors (layouts above). */
typedef struct moe_layer_weights {
  const float* router;      /* [E][H] float */
  const void* gate;         /* (E*F) x H, expert_type */
  const void* up;           /* (E*F) x H, expert_type */
  const void* down;         /* (E*H) x F, down_type (0: expert_type) */
  const void* shared_gate;  /* Fs x H, shared_type (unused if Fs == 0) */
  const void* shared_up;    /* Fs x H, shared_type */
  const void* shared_down;  /* H x Fs, shared_type */
} moe_layer_weights;

/* Library version, major*10000 + minor*100 + patch. */
int32_t moe_version(void);

/* Human-readable text of a status code (static string, never NULL). */
const char* moe_strerror(int32_t status);

/* Bytes of a rows x cols tensor of `dtype` in the layout above, in *bytes.
 * MOE_ERR_DTYPE for an unknown type, MOE_ERR_SHAPE if cols does not fit
 * the block size or rows/cols are negative. */
int32_t moe_tensor_bytes(int32_t dtype, int64_t rows, int64_t cols, int64_t* bytes);

/* Device workspace, in *bytes, that moe_layer_forward and moe_route need for
 * up to max_tokens tokens: hand-off areas, router logits, routing lists,
 * the SwiGLU activations of every (token, slot) pair, the per-pair expert
 * outputs, and for batches above 16 tokens the split activations and the
 * token-tile list of the grouped GEMMs.  The hand-off areas at the start
 * (16384 bytes of counters, then E*64 bytes of routing keys rounded up to a
 * multiple of 256) must be zero before the first call that uses the
 * workspace; every call leaves them zero again, so zero-fill a workspace
 * once when it is allocated.  Calls that share a workspace must not overlap
 * in time.  The routing step of calls of up to 16 tokens waits, with a
 * bounded poll, for router results of workgroups that the GPU dispatches
 * before it, so the wait always ends in normal operation; if it ever gave
 * up, that call's routing weights (and so its outputs) are NaN and the
 * first 32-bit word of the workspace is set nonzero (the kernels never read
 * it; the caller may check and clear it). */
int32_t moe_workspace_bytes(const moe_layer_desc* desc, int32_t max_tokens, size_t* bytes);

/* Routing only (steps: router GEMV, top-k with renormalised softmax weights,
 * per-expert bucketing).  Outputs (device, caller-allocated):
 *   topk_ids [M][k] int32, topk_w [M][k] float,
 *   expert_counts [E] int32 (pairs routed to each expert),
 *   expert_offsets [E+1] int32 (exclusive prefix sums of counts),
 *   token_slots [M*k] int32: for each expert in ascending order, the pair
 *     indices p = t*k + j routed to it, t ascending,
 *   active_experts [E] int32: experts with count > 0, ascending, then -1,
 *   n_active [1] int32: their number.
 * Any output except topk_ids/topk_w may be NULL. */
int32_t moe_route(const moe_layer_desc* desc, const float* router, const float* x,
                  int32_t n_tokens, int32_t* topk_ids, float* topk_w,
                  int32_t* expert_counts, int32_t* expert_offsets, int32_t* token_slots,
                  int32_t* active_experts, int32_t* n_active,
                  void* workspace, size_t workspace_bytes, void* hip_stream);

/* The whole layer: y [M][H] float from x [M][H] float.  topk_ids [M][k] and
 * topk_w [M][k] receive the routing if non-NULL.  workspace must hold
 * moe_workspace_bytes(desc, n_tokens) bytes (device, 256-byte aligned,
 * counter page zero as described above).
 * Calls of up to 16 tokens run three stages
 * ("route_shared_gateup", "gateup", "down_combine").  Larger batches (a
 * prefill micro-batch, "Step-5 Preview GGUF": 512-token micro-batches) run
 * the expert FFNs as grouped GEMMs on the bf16 matrix cores with exact
 * integer quants, fp32 scales and activations split into two bf16 terms,
 * in five stages ("route", "shared_gateup", "gateup", "shared_down",
 * "down_combine"; the shared stages are empty without a shared expert),
 * for every routed type and pairing of gate/up and down types.
 * moe_stage_count / moe_stage_name say which. */
int32_t moe_layer_forward(const moe_layer_desc* desc, const moe_layer_weights* weights,
                          const float* x, int32_t n_tokens, float* y,
                          int32_t* topk_ids, float* topk_w,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_layer_forward without a workspace argument.  The workspace is a
 * device array inside the library of MOE_NOALLOC_MAX_WORKSPACE bytes, one
 * per GPU, held until the process ends; the call allocates nothing (no
 * hipMalloc, no hipFree).  A call whose moe_workspace_bytes(desc, n_tokens)
 * exceeds MOE_NOALLOC_MAX_WORKSPACE returns MOE_ERR_WORKSPACE before
 * enqueueing anything (at H = 4096 batches up to 16 tokens fit; 512-token
 * prefill batches do not).  The first call on a device looks up the array's
 * address and clears its counter page on hip_stream.  Every call on a GPU
 * shares that GPU's array, so calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 * Arguments, outputs and the other status codes are those of
 * moe_layer_forward. */
#define MOE_NOALLOC_MAX_WORKSPACE (8u << 20)
int32_t moe_layer_forward_noalloc(const moe_layer_desc* desc, const moe_layer_weights* weights,
                                  const float* x, int32_t n_tokens, float* y,
                                  int32_t* topk_ids, float* topk_w, void* hip_stream);

/* Number of stages a moe_layer_forward call with this desc and n_tokens
 * enqueues (1, 3 or 5; the negated status code if desc is invalid), and the
 * name of stage i (static string; NULL if i or desc is invalid). */
int32_t moe_stage_count(const moe_layer_desc* desc, int32_t n_tokens);
const char* moe_stage_name(const moe_layer_desc* desc, int32_t n_tokens, int32_t i);

/* moe_layer_forward that also records events[i] (hipEvent_t, created by the
 * caller) on hip_stream before stage i and events[n] after the last stage,
 * n = moe_stage_count(desc, n_tokens), so that the caller can time each
 * stage.  A NULL entry is skipped (no event recorded at that boundary).
 * n_events must be n + 1, else MOE_ERR_ARG. */
int32_t moe_layer_forward_timed(const moe_layer_desc* desc, const moe_layer_weights* weights,
                                const float* x, int32_t n_tokens, float* y,
                                int32_t* topk_ids, float* topk_w,
                                void* workspace, size_t workspace_bytes, void* hip_stream,
                                void* const* events, int32_t n_events);

/* Dequantise rows [row_start, row_start + row_count) of a rows x cols tensor
 * of `dtype` into out [row_count][cols] float (test hook for the block
 * decoders).  Q8_0 yields d*q, Q4_K and Q2_K yield fma(d*sc, q, -(dmin*m)),
 * Q3_K yields (d*(S-32))*(Q-4), Q6_K (d*sc)*(Q-32); all are the exactly
 * rounded float of the block's value. */
int32_t moe_dequant_rows(int32_t dtype, const void* tensor, int64_t rows, int32_t cols,
                         int64_t row_start, int64_t row_count, float* out, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SVR_MOE_LAYER_H */
