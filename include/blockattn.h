/*
 * blockattn.h -- C ABI of the exact blockwise causal attention library (gfx950).
 *
 * The operation: exact softmax attention of a resident block of queries against
 * key/value chunks taken in any order, with each chunk's partial result carried
 * as a per-row pair (O, LSE) and pairs merged so that the final result equals
 * attention over all keys at once.  This is one host's step of Ring Attention
 * ("Ring Attention with Blockwise Transformers for Near-Infinite Context",
 * research.elamur.ai summary, section Summary: each host keeps its query block,
 * key/value blocks arrive one at a time, the result does not depend on the order
 * and attention stays exact).  LongLoRA's shifted sparse attention
 * ("LongLoRA: Efficient Fine-tuning of Long-Context Large Language Models",
 * research.elamur.ai summary, sections Summary and Key points) is a mask mode of
 * the same kernels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or synchronises, and keeps no pointer past return.
 *  - Work is enqueued on `stream` (0 = the default stream) and is asynchronous;
 *    a fault inside a kernel surfaces at the caller's next synchronisation.
 *  - All arguments are validated before anything is enqueued; on any error
 *    nothing is enqueued and a positive ba_status is returned.
 *  - Layouts: query-shaped tensors (q, o, o_final, dout, dq_acc, dq_final) are
 *    [B, Sq, Hq, D]; key-shaped tensors (k, v, dk, dv) are [B, Sk, Hkv, D].  The
 *    D axis is contiguous (stride 1); the b, s, h strides are given in ELEMENTS
 *    in ba_desc and must be non-negative multiples of 8: q_stride for q,
 *    o_stride for every other query-shaped tensor (o, o_final, dout, dq_acc,
 *    dq_final; in lse_merge o_acc, o_part, o_final), kv_stride for every
 *    key-shaped one.  So q may be a strided view (say a slice of a packed
 *    [B, S, 3, H, D] projection) while the outputs are dense, or the reverse.
 *    Row statistics (lse, delta) are dense fp32 [B, Hq, Sq].
 *  - Pointers to bf16/fp32 tensors must be 16-byte aligned; lse/delta 4-byte.
 *  - Dtypes: q, k, v, dout are bf16.  LSE, delta and accumulators are fp32.
 *    Every bf16 store rounds to nearest even.
 *  - Positions: query row i sits at global position q_pos0 + i and key row j at
 *    k_pos0 + j.  With causal = 1, key j is allowed for query i iff
 *    k_pos0 + j <= q_pos0 + i (the diagonal is included).
 *  - LSE is the natural log of the sum of exp of the SCALED scores of the
 *    allowed keys; a row with no allowed key has the pair (O, LSE) = (0, -inf),
 *    which every merge treats as the identity.
 *  - The library is stateless, re-entrant and thread-safe.
 */
#ifndef BLOCKATTN_H
#define BLOCKATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BA_OK = 0,
  BA_ERR_NULL = 1,        /* a required pointer is NULL */
  BA_ERR_SHAPE = 2,       /* negative size, heads_q % heads_kv != 0, ... */
  BA_ERR_STRIDE = 3,      /* a b/s/h stride is negative or not a multiple of 8 elements,
                             or a sequence (s) stride is 2^24 elements or more */
  BA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned (lse/delta: 4-byte) */
  BA_ERR_UNSUPPORTED = 5, /* head_dim not in {64, 128}, or an unknown dtype */
  BA_ERR_S2 = 6,          /* invalid S2 layout (see ba_s2_desc) */
  BA_ERR_MODE = 7,        /* unknown mode/flags, or ACCUMULATE with a non-fp32 o */
  BA_ERR_LAUNCH = 8,      /* the HIP runtime rejected a launch */
  BA_ERR_WORKSPACE = 9    /* blockattn_bwd_noalloc: the problem exceeds the static scratch buffer */
} ba_status;

typedef enum { BA_F32 = 0, BA_BF16 = 1 } ba_dtype;

typedef enum {
  BA_OVERWRITE = 0,  /* (o, lse) := this chunk's partial pair, for EVERY query row */
  BA_ACCUMULATE = 1, /* (o, lse) := merge((o, lse), partial); rows the chunk cannot reach are untouched */
  /* Flag OR-ed into either mode of blockattn_fwd: with o_final, store the final
   * output only for the query tiles the chunk reaches and leave the rows of the
   * others untouched (no conversion of them from o).  For a causal ring whose
   * caller passes o_final on each step that is the last one to reach some rows
   * (the step's chunk precedes every later step's chunk), every row's final
   * output is stored by that step. */
  BA_FINAL_REACHED_ONLY = 4
} ba_mode;

typedef enum {
  BA_BWD_COMPUTE_DELTA = 1, /* first compute delta = rowsum(dout * o) into `delta` */
  BA_BWD_FINALIZE_DQ = 2    /* last convert dq_acc to bf16 into `dq_final` */
} ba_bwd_flags;

typedef struct {
  int32_t batch;      /* B >= 0 */
  int32_t heads_q;    /* Hq >= 1 */
  int32_t heads_kv;   /* Hkv >= 1, Hq % Hkv == 0; query head h reads key/value head h / (Hq / Hkv) */
  int32_t head_dim;   /* D in {64, 128} */
  int64_t seqlen_q;   /* Sq >= 0: rows of the resident query block */
  int64_t seqlen_k;   /* Sk >= 0: rows of this key/value chunk */
  int64_t q_pos0;     /* global position of query row 0 */
  int64_t k_pos0;     /* global position of key row 0 (the ring step's chunk offset) */
  int32_t causal;     /* 1: causal mask on global positions; 0: every key allowed */
  float scale;        /* softmax scale; <= 0 selects 1/sqrt(head_dim); the forward and backward
                         return BA_ERR_SHAPE for NaN or inf */
  int64_t q_stride[3];  /* (b, s, h) element strides of q */
  int64_t kv_stride[3]; /* (b, s, h) element strides of every key-shaped tensor (k, v, dk, dv) */
  int64_t o_stride[3];  /* (b, s, h) element strides of every other query-shaped tensor
                           (o, o_final, dout, dq_acc, dq_final; lse_merge: all of its tensors) */
} ba_desc;

/* S2-Attn layout (LongLoRA summary, Summary: tokens split into groups, attention
 * inside each group, half of the heads shifted by half a group; Key points:
 * group 2048 for 8192-token training).  Heads [shift_head0, Hq) are rolled so
 * that rolled position r holds original position (r + group/2) mod S, attend
 * causally inside groups of `group` rolled positions, and are stored back at
 * their original rows; heads [0, shift_head0) attend causally inside groups of
 * original positions.  Requirements (else BA_ERR_S2): seqlen_q == seqlen_k = S,
 * q_pos0 == k_pos0 == 0, causal == 1, group even, S % group == 0,
 * (group / 2) % 256 == 0 (a query tile never straddles the roll), 0 <= shift_head0
 * <= Hq and shift_head0 % (Hq / Hkv) == 0 (a key/value head is either shifted
 * for all of its query heads or for none). */
typedef struct {
  int32_t group;
  int32_t shift_head0;
} ba_s2_desc;

/* Forward of one ring step: attention of the query block (q) against one key/
 * value chunk (k, v: seqlen_k rows at global offset k_pos0), producing the
 * chunk's partial pair and (ACCUMULATE) merging it into the running pair.
 *   o        [B,Sq,Hq,D], o_dtype BA_F32 or BA_BF16 (BA_ACCUMULATE needs BA_F32):
 *            OVERWRITE: out; ACCUMULATE: in/out running normalised output.
 *   lse      [B,Hq,Sq] fp32, same in/out role as o.
 *   o_final  optional (NULL): bf16 [B,Sq,Hq,D] receives the normalised output of
 *            EVERY row after this step (rows the chunk cannot reach are converted
 *            from o), so the last ring step also produces the final result; with
 *            BA_FINAL_REACHED_ONLY in mode, only the rows of the query tiles the
 *            chunk reaches.
 * Defined by the Ring Attention summary (Summary): blockwise attention of a
 * resident query block, combinable in any block order. */
int blockattn_fwd(const ba_desc* desc, const void* q, const void* k, const void* v,
                  void* o, int32_t o_dtype, float* lse, int32_t mode, void* o_final,
                  hipStream_t stream);

/* Standalone merge of partial pairs: (o_acc, lse_acc) := merge((o_acc, lse_acc),
 * (o_part, lse_part)) for every row, with
 *   L = log(e^La + e^Lb),  O = e^(La - L) O_a + e^(Lb - L) O_b,
 * a pair with LSE = -inf contributing nothing whatever its O holds, and two
 * such pairs giving (0, -inf).  Uses batch, heads_q, head_dim, seqlen_q and
 * o_stride of desc (shared by o_acc, o_part and o_final).  o_acc is fp32;
 * o_part is fp32 or bf16 (part_dtype); o_final (nullable) receives bf16 of the
 * merged output.  Same source as
 * blockattn_fwd (order-independent combination of blocks). */
int lse_merge(const ba_desc* desc, float* o_acc, float* lse_acc, const void* o_part,
              int32_t part_dtype, const float* lse_part, void* o_final, hipStream_t stream);

/* Backward of one ring step: the gradient of <dout, O> where O is the FINAL
 * attention output (all chunks) and lse its final LSE.
 *   o, dout  bf16 [B,Sq,Hq,D] final output and upstream gradient.
 *   lse      fp32 [B,Hq,Sq] final LSE.
 *   delta    fp32 [B,Hq,Sq]: written when flags has BA_BWD_COMPUTE_DELTA
 *            (delta_i = sum_d dout_id * o_id), read otherwise.
 *   dq_acc   fp32 [B,Sq,Hq,D], accumulated (+=): the caller zeroes it before
 *            the first ring step.
 *   dk, dv   [B,Sk,Hkv,D] of this chunk, dtype dkv_dtype (BA_F32 or BA_BF16),
 *            overwritten; for GQA each key/value head gets the sum over its
 *            query heads.
 *   dq_final optional bf16 [B,Sq,Hq,D]: written from dq_acc after this step's
 *            contribution when flags has BA_BWD_FINALIZE_DQ.
 * With S = tau Q K^T, P = exp(S - LSE), dP = dout V^T, dS = P (dP - delta):
 * dV = P^T dout, dK = tau dS^T Q, dQ = tau dS K.  The pages train with this
 * attention (project page "How It Works"; LongLoRA and Ring Attention
 * summaries) without printing the gradient; this is the analytic one. */
int blockattn_bwd(const ba_desc* desc, const void* q, const void* k, const void* v,
                  const void* o, const void* dout, const float* lse, float* delta,
                  float* dq_acc, void* dk, void* dv, int32_t dkv_dtype, void* dq_final,
                  int32_t flags, hipStream_t stream);

/* Allocation-free variant of blockattn_bwd, for callers that cannot allocate
 * device memory or take workspace arguments (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Arguments and results
 * as blockattn_bwd without `delta`: the delta rows live in a static device
 * buffer of the library (`scratch`, BLOCKATTN_NOALLOC_MAX_ROWS fp32 values =
 * 32 MiB, one per GPU, held until the process ends) and are computed on EVERY
 * call (BA_BWD_COMPUTE_DELTA is implied; FINALIZE_DQ is honoured), so each call
 * stands alone and its outputs equal blockattn_bwd's bit for bit.  The buffer
 * of the calling thread's current device (hipGetDevice) is used; every call on
 * that GPU shares it, so calls that overlap on one GPU (other streams, other
 * threads) race.  Calls no hipMalloc/hipFree.  Errors: those of blockattn_bwd,
 * plus BA_ERR_WORKSPACE (checked before anything is enqueued) when
 * batch * heads_q * seqlen_q exceeds BLOCKATTN_NOALLOC_MAX_ROWS or the buffer's
 * device address cannot be obtained. */
#define BLOCKATTN_NOALLOC_MAX_ROWS (1LL << 23)
int blockattn_bwd_noalloc(const ba_desc* desc, const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse, float* dq_acc,
                          void* dk, void* dv, int32_t dkv_dtype, void* dq_final, int32_t flags,
                          hipStream_t stream);

/* S2-Attn forward over the whole sequence (one shot, no ring chunks):
 * o (dtype o_dtype) and lse are overwritten for every row, at original
 * positions.  See ba_s2_desc for the layout and requirements. */
int s2attn_fwd(const ba_desc* desc, const ba_s2_desc* s2, const void* q, const void* k,
               const void* v, void* o, int32_t o_dtype, float* lse, hipStream_t stream);

/* S2-Attn backward: as blockattn_bwd with the S2 mask (whole sequence, one
 * shot).  dq_acc must be zeroed by the caller; dq_final is written when
 * BA_BWD_FINALIZE_DQ is set. */
int s2attn_bwd(const ba_desc* desc, const ba_s2_desc* s2, const void* q, const void* k,
               const void* v, const void* o, const void* dout, const float* lse,
               float* delta, float* dq_acc, void* dk, void* dv, int32_t dkv_dtype,
               void* dq_final, int32_t flags, hipStream_t stream);

/* ---- Ulysses sequence parallelism: the layout permutes around its all-to-all ----
 * DeepSpeed Ulysses, one of the sequence-parallel methods the long-context
 * recipe supports beside Ring Attention (project page "How It Works"; the Ring
 * Attention summary's references), shards the sequence over N devices and
 * exchanges it for a head sharding around attention.  Device r holds
 * x = [B, Sl, H, D] (its Sl =
 * S / N rows, all heads).  These two calls are the device's local halves of the
 * exchange (the all-to-all itself needs N devices and is not here):
 *   ulysses_pack:    send[n][b][s][j][d] = x[b][s][n*(H/N) + j][d]
 *                    (send block n, [B, Sl, H/N, D], goes to device n)
 *   ulysses_unpack:  x[b][s][n*(H/N) + j][d] = recv[n][b][s][j][d]
 *                    (recv block n came from device n)
 * For B = 1, the blocks a device receives after packing, in source order, are
 * already the dense [1, S, H/N, D] tensor of its heads over the whole
 * sequence, which the attention calls take as is; the output goes back through
 * the same exchange and ulysses_unpack.
 * All tensors are dense (row-major in the index order shown), bf16, 16-byte
 * aligned; head_dim a multiple of 8; heads % n_devices == 0; src and dst must
 * not overlap.  Bit-exact copies.  Errors: BA_ERR_NULL, BA_ERR_SHAPE (negative
 * size, n_devices < 1, heads % n_devices != 0, head_dim % 8 != 0), BA_ERR_ALIGN,
 * BA_ERR_LAUNCH.  Zero-size problems return BA_OK without launching. */
int ulysses_pack(const void* x, void* send, int64_t batch, int64_t seqlen_local, int32_t heads,
                 int32_t head_dim, int32_t n_devices, hipStream_t stream);
int ulysses_unpack(const void* recv, void* x, int64_t batch, int64_t seqlen_local, int32_t heads,
                   int32_t head_dim, int32_t n_devices, hipStream_t stream);

/* ---- Blockwise feedforward (BPT) ----
 * Each host of the ring computes attention and the feedforward for its query
 * block, block by block (Ring Attention summary, Summary; the blockwise
 * parallel transformer runs the feedforward per block so the hidden activation
 * of the whole sequence never exists, Key points).  The feedforward of the
 * models the pages train (LLaMA / Llama-2) is SwiGLU:
 *   out = (silu(x W1^T) * (x W3^T)) W2^T,  silu(z) = z / (1 + exp(-z)).
 * x, out: [rows, d_model]; w1, w3: [d_ff, d_model]; w2: [d_model, d_ff]
 * (row-major, the [out, in] layout of a linear layer); hidden: caller-owned
 * workspace of at least min(block_rows, rows) x d_ff elements.  All bf16, dense,
 * 16-byte aligned.  Rows are processed in blocks of block_rows, each as two
 * launches (hidden = silu(x W1^T) * (x W3^T) rounded to bf16, then
 * out = hidden W2^T), fp32 accumulation, bf16 stores (round to nearest even).
 * Requirements: d_model % 256 == 0, d_ff % 128 == 0, every operand under 2^31
 * elements.  Errors: BA_ERR_NULL, BA_ERR_SHAPE, BA_ERR_ALIGN, BA_ERR_LAUNCH. */
int bpt_ffn(const void* x, const void* w1, const void* w3, const void* w2, void* out, void* hidden,
            int64_t rows, int32_t d_model, int32_t d_ff, int64_t block_rows, hipStream_t stream);

/* Human-readable name of a ba_status value (static storage). */
const char* blockattn_status_string(int status);

/* ---- host-side introspection (no GPU work; used by the host-logic tests) ----
 * The forward tile scheduler's enumeration of (query tile, key tile) work for
 * one (batch, head): writes up to `cap` records of 4 int64 each:
 *   {q_row0, q_rows, k_row0, k_rows}
 * (original row indices into the query block and into the key chunk) for every
 * key tile every query tile visits, in visiting order, and returns the number
 * of records (which may exceed cap), or -(ba_status) on invalid arguments.
 * s2 may be NULL.  Tile sizes are those the forward kernel uses. */
int64_t blockattn_debug_fwd_schedule(const ba_desc* desc, const ba_s2_desc* s2, int32_t head,
                                     int64_t* out, int64_t cap);

/* Tile sizes (rows) of the forward kernel's query and key tiles. */
int blockattn_debug_tile_sizes(int32_t head_dim, int32_t* block_q, int32_t* block_k);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKATTN_H */
