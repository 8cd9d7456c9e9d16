/*
 * decstep.h -- C ABI of the decode-step hot path of a Parler-TTS-style
 * multi-codebook audio-token decoder, for AMD Instinct MI355X (gfx950).
 *
 * Source: the "Optimized Parler TTS" page.  One decode step of its decoder
 * (a MusicGen-style autoregressive decoder, "A rough architecture of Parler
 * TTS") does, per layer, single-token causal self-attention over a static KV
 * cache and cross-attention over the encoded description, and ends by
 * sampling one token for each of the 9 DAC codebooks.  "Analysis and
 * improvements" keeps both caches static and preallocated so that a whole
 * step can be captured as one graph, and samples without a GPU/CPU
 * synchronisation; "Future work" asks for paged attention against the cost of
 * moving the whole static cache, and for one fused sampling kernel in place of
 * the ten-plus temperature / top-k / softmax kernels.  This library reads only
 * the valid prefix of each static cache and samples in one kernel.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *     every buffer; the library never allocates, frees, synchronises or reads
 *     device data on the host, so every call is legal inside hip stream
 *     capture.  All work is enqueued on `stream` (a hipStream_t, may be NULL
 *     for the default stream) and is asynchronous.
 *   - Layouts are row-major and contiguous.  bf16 tensors hold IEEE bfloat16
 *     bit patterns.  q, k, v and the workspace must be 16-byte aligned, every
 *     other device pointer 4-byte aligned.
 *   - The return value is a dec_status.  Problems visible on the host are
 *     reported before anything is enqueued (nothing is launched, no HIP call
 *     is made).  DEC_E_HIP means a HIP call failed; dec_last_hip_error()
 *     returns its hipError_t (per calling thread).
 *   - Values that live on the device cannot be checked on the host; they have
 *     defined results instead (stated per function).
 */
#ifndef DECSTEP_H
#define DECSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dec_stream_t;   /* the same type as hipStream_t */

enum dec_dtype { DEC_BF16 = 0, DEC_F32 = 1 };

enum dec_status {
  DEC_OK = 0,
  DEC_E_NULL = 1,         /* a required pointer is NULL */
  DEC_E_SHAPE = 2,        /* a size is out of range or sizes disagree */
  DEC_E_DTYPE = 3,        /* unknown dtype code */
  DEC_E_WORKSPACE = 4,    /* workspace smaller than dec_attn_workspace_bytes() */
  DEC_E_UNSUPPORTED = 5,  /* a legal but unimplemented case (e.g. head_dim other than 64 or 128) */
  DEC_E_HIP = 6,          /* a HIP runtime call failed */
  DEC_E_ALIGN = 7         /* a pointer is not aligned as required */
};

/* Keys per split-K chunk of the attention kernels: the largest chunk, 1024.
 * A sequence of n valid keys is cut into ceil(n / chunk) chunks; each chunk's
 * partial softmax state (max, sum, weighted values) is formed in a fixed order
 * and the chunk states fold in chunk order.  A launch with few sequences,
 * whose chunks (counted at full capacity) would give fewer than one work item
 * per four CUs, halves the chunk (down to 128 keys) until they do, when its
 * workspace holds the chunk states at 128 keys (dec_attn_workspace_bytes
 * sizes it so).  A launch that gives each sequence one workgroup also cuts
 * the excess of its heaviest sequences in halves: when the sequences of the
 * longest length (each one chunk, of more than half a chunk) number a multiple
 * of the CU count plus E, with E at least a quarter of the CU count, the last E
 * of the longest group become two half-chunk items each, so the CUs carry
 * nearly equal bytes.  The cut therefore depends on n, the call's shape and
 * capacities, the workspace size and the device's CU count, never on the grid
 * or on how chunks are spread over workgroups: results are bitwise
 * reproducible for a given call on a given device. */
int dec_attn_chunk_keys(void);

/* Workspace bytes for attention over n_layers x B x H sequences with a self
 * cache of L_cap_self slots and a cross cache of L_cap_cross slots (pass 0 for
 * a cache that the call does not use).  It holds two regions of per-sequence
 * arrival counters (a call's first and second cache) and the chunk states used
 * when a launch spreads a sequence's chunks over several workgroups (launches
 * with few sequences do), sized for 128-key chunks; capacities of at most 128
 * slots need none.  A call also accepts a smaller workspace that holds the
 * states at 1024-key chunks (none when its capacities fit 1024 slots), and
 * then keeps 1024-key chunks.  One workspace sized for both caches serves
 * dec_attn_self, dec_attn_cross and dec_attn_step of one n_layers x B x H
 * shape; calls of another shape need their own workspace, or
 * dec_attn_workspace_init in between.  The size returned also holds, after the
 * counters and states, 256 KiB of first-tile records: every wave of a launch
 * records which tile it read first, and the next launch on the workspace
 * requests that tile at once, before it has derived its own schedule, and
 * keeps it only when its first tile is the same one (the address comes from the
 * call's own arguments and is checked against them, so a record left by any
 * other call costs at most bytes read in vain).  In dec_attn_step_append a record
 * one key shorter also serves: that key is the current token's, taken from the
 * new rows.  A workspace without room for
 * the records runs without them; outputs are the same bit for bit.  Returns 0
 * on bad sizes. */
size_t dec_attn_workspace_bytes(int n_layers, int B, int H, int hd,
                                int L_cap_self, int L_cap_cross);

/* Zero a workspace with a fill kernel (capturable).  Required once after
 * allocation: the arrival counters must start at zero, and every attention
 * call leaves them at zero again when it completes.  Calls that share one
 * workspace must be ordered (same stream); concurrent use of one workspace
 * races. */
int dec_attn_workspace_init(void* workspace, size_t ws_bytes, dec_stream_t stream);

/* Single-token self-attention over the valid prefix of a static KV cache
 * ("Analysis and improvements": static caches for causal attention; only the
 * valid prefix is read, unlike the whole-cache transfer described there).
 *
 *   q    [n_layers, B, H, hd]          dtype
 *   k, v [n_layers, B, H, L_cap, hd]   dtype; slots >= len[b] are never read
 *   len  [B] int32, valid slots of sequence b INCLUDING the current token
 *   out  [n_layers, B, H, hd] float32:
 *          out = sum_j softmax_j(scale * <q, k_j>) v_j   over j < len[b]
 *   hd is 64 (the model's head size) or 128; dtype is DEC_BF16 or DEC_F32;
 *   accumulation is float32.  One sequence's cache, L_cap * hd * element
 *   size, must stay below 2 GiB (else DEC_E_UNSUPPORTED).
 * Device-side values: len[b] <= 0 gives an all-zero output row; len[b] >
 * L_cap is read as L_cap.  n_layers > 1 means layer-stacked buffers served by
 * one launch.  B is at most 4096 (2048 for dec_attn_step): DEC_E_UNSUPPORTED. */
int dec_attn_self(const void* q, const void* k, const void* v, const int32_t* len,
                  float* out, int n_layers, int B, int H, int L_cap, int hd, int dtype,
                  float scale, void* workspace, size_t ws_bytes, dec_stream_t stream);

/* Cross-attention over the encoded description ("A rough architecture of
 * Parler TTS": the description states feed cross-attention in the decoder;
 * "Analysis and improvements": the static cross-attention cache).  Same
 * arguments as dec_attn_self with enc_len [B] (valid description states) in
 * place of len and L_cap the description capacity. */
int dec_attn_cross(const void* q, const void* k, const void* v, const int32_t* enc_len,
                   float* out, int n_layers, int B, int H, int L_cap, int hd, int dtype,
                   float scale, void* workspace, size_t ws_bytes, dec_stream_t stream);

/* Self-attention and cross-attention of the same step in ONE launch: equal to
 * dec_attn_self(q_self, ...) followed by dec_attn_cross(q_cross, ...), bit for
 * bit, except where the halving above sees different heavy sequences in the
 * joint launch than in the separate ones (both caches at the longest length);
 * those outputs differ in rounding only, within the same bars.  workspace must
 * hold dec_attn_workspace_bytes(n_layers, B, H, hd, L_cap_self, L_cap_cross)
 * bytes. */
int dec_attn_step(const void* q_self, const void* k_self, const void* v_self,
                  const int32_t* len, int L_cap_self, float* out_self,
                  const void* q_cross, const void* k_cross, const void* v_cross,
                  const int32_t* enc_len, int L_cap_cross, float* out_cross,
                  int n_layers, int B, int H, int hd, int dtype, float scale,
                  void* workspace, size_t ws_bytes, dec_stream_t stream);

/* dec_attn_step with the current token's key and value rows appended to the
 * static self cache in the same launch ("Analysis and improvements": the
 * cache is preallocated and a step writes its next row; the whole step is
 * one graph).  k_new, v_new [n_layers, B, H, hd] dtype, 16-byte aligned.
 * For a sequence with 1 <= len[b] <= L_cap_self, self-attention uses k_new /
 * v_new as key len[b] - 1 and the launch writes them to that slot of k_self /
 * v_self; with len[b] < 1 or len[b] > L_cap_self nothing is written and the
 * cache is read as it is.  Outputs and caches equal those of dec_kv_append
 * followed by dec_attn_step bit for bit; one launch instead of two.  Other
 * arguments, errors and the workspace as dec_attn_step. */
int dec_attn_step_append(const void* q_self, void* k_self, void* v_self, const int32_t* len,
                         int L_cap_self, float* out_self, const void* k_new, const void* v_new,
                         const void* q_cross, const void* k_cross, const void* v_cross,
                         const int32_t* enc_len, int L_cap_cross, float* out_cross, int n_layers,
                         int B, int H, int hd, int dtype, float scale, void* workspace,
                         size_t ws_bytes, dec_stream_t stream);

/* For callers that cannot allocate device memory (code under stream capture
 * that may not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation): dec_attn_step without a workspace argument.  The arrival
 * counters and chunk states live in a library-owned device array of
 * DEC_NOALLOC_SCRATCH_BYTES bytes (one per GPU, held until the process
 * ends); the call allocates and frees nothing.  The first call on a device
 * takes the array's address there (a HIP symbol lookup, no allocation).
 * Every call clears the array's arrival counters with a fill kernel on
 * `stream` before the attention launch, so a call starts from zero whatever
 * the previous one left.  The layout is the one a workspace of that size
 * gets from dec_attn_step (the chunk states at 128 keys when they fit, else
 * at 1024 keys), so outputs equal dec_attn_step's with such a workspace bit
 * for bit.  A shape whose states fit neither way (dec_attn_workspace_bytes
 * at 1024-key chunks above the array's size) returns DEC_E_WORKSPACE before
 * anything is enqueued.  All calls on one GPU share the array: calls that
 * overlap on a device (other streams, other threads) race and must be
 * ordered by the caller.  Everything else as dec_attn_step. */
#define DEC_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int dec_attn_step_noalloc(const void* q_self, const void* k_self, const void* v_self,
                          const int32_t* len, int L_cap_self, float* out_self,
                          const void* q_cross, const void* k_cross, const void* v_cross,
                          const int32_t* enc_len, int L_cap_cross, float* out_cross,
                          int n_layers, int B, int H, int hd, int dtype, float scale,
                          dec_stream_t stream);

/* dec_attn_step with two widenings (both optional):
 *   cross_mask  [B, mask_words] uint32, or NULL: an arbitrary boolean mask over
 *               the description ("A rough architecture of Parler TTS": the
 *               encoded description feeds cross-attention; padding inside it is
 *               hidden by an attention mask).  Bit j % 32 of word j / 32 of row b
 *               set = key j attended.  Keys j < enc_len[b] with their bit set
 *               take part; a row with none outputs zeros.  mask_words must be
 *               even and at least 2 * ceil(L_cap_cross / 64) (a tile reads the
 *               whole words that hold its keys' bits); 8-byte aligned.  A tile
 *               with no attended key is not read; the other keys of a tile that
 *               has one are read and weighted zero, so masked keys below
 *               enc_len[b] must hold finite values.
 *   out_dtype   DEC_F32 (float outputs, as dec_attn_step) or DEC_BF16 (outputs
 *               rounded to bfloat16, nearest-even, from the same fp32 values;
 *               out pointers 2-byte aligned).
 * Everything else as dec_attn_step. */
int dec_attn_step_ex(const void* q_self, const void* k_self, const void* v_self,
                     const int32_t* len, int L_cap_self, void* out_self, const void* q_cross,
                     const void* k_cross, const void* v_cross, const int32_t* enc_len,
                     const uint32_t* cross_mask, int mask_words, int L_cap_cross,
                     void* out_cross, int n_layers, int B, int H, int hd, int dtype,
                     int out_dtype, float scale, void* workspace, size_t ws_bytes,
                     dec_stream_t stream);

/* Self-attention over a PAGED cache ("Future work": paged attention, so a
 * sequence's keys live in fixed-size blocks drawn from a shared pool instead of
 * one preallocated run of L_cap slots).  Same arithmetic as dec_attn_self; only
 * the address of each key changes, so for equal logical contents the outputs are
 * bit-identical to dec_attn_self.
 *
 *   q            [n_layers, B, H, hd]                         dtype
 *   k_pool,
 *   v_pool       [n_layers, n_blocks, H, block_size, hd]      dtype
 *   block_table  [B, max_blocks] int32: key j of sequence b is row j % block_size
 *                of physical block block_table[b][j / block_size] (the same
 *                table for every layer and head)
 *   len          [B] int32, clamped to [0, max_blocks * block_size]
 *   out          [n_layers, B, H, hd] float32
 * block_size: a power of two, at least 64 (a tile, 32 keys at hd 64 and 16 at
 * hd 128, never crosses a block),
 * else DEC_E_UNSUPPORTED.  Workspace: dec_attn_workspace_bytes with
 * L_cap_self = max_blocks * block_size.  Device-side: a table entry outside
 * [0, n_blocks) makes that block read as zero rows (nothing outside the pool is
 * touched); entries past ceil(len[b] / block_size) are never read. */
int dec_attn_self_paged(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* len, float* out,
                        int n_layers, int B, int H, int hd, int block_size, int n_blocks,
                        int max_blocks, int dtype, float scale, void* workspace,
                        size_t ws_bytes, dec_stream_t stream);

/* dec_attn_step with the self-attention cache paged (as dec_attn_self_paged) and
 * the description cache static, in one launch. */
int dec_attn_step_paged(const void* q_self, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* len, int block_size,
                        int n_blocks, int max_blocks, float* out_self, const void* q_cross,
                        const void* k_cross, const void* v_cross, const int32_t* enc_len,
                        int L_cap_cross, float* out_cross, int n_layers, int B, int H, int hd,
                        int dtype, float scale, void* workspace, size_t ws_bytes,
                        dec_stream_t stream);

/* dec_attn_step_paged with the widenings of dec_attn_step_ex: a boolean key
 * mask over the (static) description cache and fp32 or bf16 outputs, in one
 * launch.  The self cache is paged as in dec_attn_self_paged (it takes no
 * mask); cross_mask, mask_words and out_dtype as in dec_attn_step_ex.  With
 * the same keys, lengths and mask, outputs equal dec_attn_step_ex's bit for bit. */
int dec_attn_step_paged_ex(const void* q_self, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const int32_t* len, int block_size,
                           int n_blocks, int max_blocks, void* out_self, const void* q_cross,
                           const void* k_cross, const void* v_cross, const int32_t* enc_len,
                           const uint32_t* cross_mask, int mask_words, int L_cap_cross,
                           void* out_cross, int n_layers, int B, int H, int hd, int dtype,
                           int out_dtype, float scale, void* workspace, size_t ws_bytes,
                           dec_stream_t stream);

/* Fused temperature / top-k / softmax / sampling of the next token of every
 * codebook, with the codebook delay mask ("Future work", item 2: one kernel in
 * place of the temperature, top-k and softmax kernels; "Analysis and
 * improvements": logits of the last position only, vocabulary padded to a
 * multiple of 8, sampling without a GPU/CPU synchronisation; "A rough
 * architecture of Parler TTS": 9 codebooks under a delay pattern).
 *
 *   logits      [B, n_cb, V_stride] float32; only columns < V_valid are read
 *   temperature [B] float32; T <= 0 selects greedy argmax
 *   top_k       1..64 (a row keeps min(top_k, V_valid) entries)
 *   uniforms    [B, n_cb] float32 in [0, 1)
 *   step        [B] int32 steps already taken, or NULL for no delay mask
 *   tokens      [B, n_cb] int32 out
 *   topk_idx    [B, n_cb, top_k] int32 out or NULL: the kept vocabulary indices
 *               in ascending order, -1 past min(top_k, V_valid)
 *   topk_prob   [B, n_cb, top_k] float32 out or NULL: their probabilities
 *               (one-hot on the chosen entry when T <= 0), 0 past the end
 * Per row: keep the min(top_k, V_valid) largest logits (equal values: the
 * lower index first); p_i = exp((x_i - max) / T) normalised over the kept set;
 * walking the kept set in ascending vocabulary order, the token is the first
 * index whose running sum of p exceeds u (the last kept index if none does).
 * If step != NULL and step[b] < c, codebook c emits fill_token instead.
 * Device-side values: non-finite logits or temperatures are outside the
 * contract but still yield an index in [0, V_valid) or fill_token. */
int dec_sample_topk(const float* logits, int B, int n_cb, int V_valid, int V_stride,
                    const float* temperature, int top_k, const float* uniforms,
                    const int32_t* step, int32_t fill_token, int32_t* tokens,
                    int32_t* topk_idx, float* topk_prob, dec_stream_t stream);

/* As dec_sample_topk, but the uniform of row (b, c) is generated on the device
 * instead of read, so a captured step needs no random numbers from the host
 * ("Analysis and improvements": sampling without a GPU/CPU synchronisation).
 * Generator: Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC 2011) at counter
 * (step[b], b, c, 0) and key (seed, 0); u = (word0 >> 40) * 2^-24, in [0, 1).
 * step == NULL: counter step 0 for every row and no delay mask, so equal calls
 * give equal tokens.  Arguments, outputs and errors otherwise as
 * dec_sample_topk (there is no uniforms argument). */
int dec_sample_topk_philox(const float* logits, int B, int n_cb, int V_valid, int V_stride,
                           const float* temperature, int top_k, uint64_t seed,
                           const int32_t* step, int32_t fill_token, int32_t* tokens,
                           int32_t* topk_idx, float* topk_prob, dec_stream_t stream);

/* Widened sampler ("Future work", item 2, as dec_sample_topk).
 *
 *   logits        [B, n_cb, V_stride], logits_dtype DEC_F32 (4-byte aligned) or
 *                 DEC_BF16 (2-byte aligned); a bf16 value widens exactly to
 *                 float32 and is then treated as dec_sample_topk treats it
 *   top_k         1..V_valid-or-more: any top_k >= 1 up to 4096 (a row keeps
 *                 min(top_k, V_valid) entries, so top_k >= V_valid keeps the
 *                 whole row); topk_idx / topk_prob hold top_k entries per row
 *   uniforms      [B, n_cb] float32 in [0, 1), or NULL: then row (b, c) draws
 *                 its uniform from Philox4x64-10 with `seed` exactly as
 *                 dec_sample_topk_philox does
 * Rule, outputs, delay mask and device-side behaviour as dec_sample_topk.  For
 * top_k <= 64 the kernel is dec_sample_topk's; above it the same arithmetic runs
 * over the kept entries 64 at a time in vocabulary order.  Both form the weights
 * exp((x - max) / T) and their sum in float64, round each probability once to
 * float32 (what topk_prob holds), and compare u with the float64 running sum of
 * those probabilities. */
int dec_sample_topk_ex(const void* logits, int logits_dtype, int B, int n_cb, int V_valid,
                       int V_stride, const float* temperature, int top_k, const float* uniforms,
                       uint64_t seed, const int32_t* step, int32_t fill_token, int32_t* tokens,
                       int32_t* topk_idx, float* topk_prob, dec_stream_t stream);

/* The widened sampler with the step's state advance in the same launch, so a
 * captured decode step needs no separate advance node ("Analysis and
 * improvements": the step is one graph with nothing left for the host).
 * Sampling, arguments, outputs and errors as dec_sample_topk_ex, except:
 *   step  [B, n_cb] int32, required (DEC_E_NULL): one counter per row, every
 *         row of sequence b holding the sequence's step (the delay mask and the
 *         Philox counter read row (b, c)'s own counter); the launch adds one to
 *         each, so no row reads a counter another row writes
 *   len   [B] int32 or NULL: the launch adds one to len[b] (the self-attention
 *         length of the next step); 4-byte aligned
 * After the launch every step counter and every len[b] is one larger; tokens,
 * top-k sets and probabilities equal those of dec_sample_topk_ex with step[b]
 * = the counters' value.  Calls on one state must be stream-ordered. */
int dec_sample_topk_advance(const void* logits, int logits_dtype, int B, int n_cb, int V_valid,
                            int V_stride, const float* temperature, int top_k,
                            const float* uniforms, uint64_t seed, int32_t* step, int32_t* len,
                            int32_t fill_token, int32_t* tokens, int32_t* topk_idx,
                            float* topk_prob, dec_stream_t stream);

/* Write the current token's key and value rows into the static caches
 * ("Analysis and improvements": caches preallocated at a fixed capacity, so a
 * step writes the next row instead of growing a tensor).
 *
 *   k_new, v_new     [n_layers, B, H, hd]          dtype, read
 *   k_cache, v_cache [n_layers, B, H, L_cap, hd]   dtype, row len[b] - 1 written
 *   len              [B] int32, read: the length INCLUDING the current token
 *                    (the value dec_attn_self reads afterwards)
 * Nothing is written for a sequence with len[b] < 1 or len[b] > L_cap.  Every
 * pointer is a device pointer owned by the caller; caches and new rows must be
 * 16-byte aligned and hd * sizeof(element) a multiple of 16 (else
 * DEC_E_ALIGN / DEC_E_UNSUPPORTED).  dtype: DEC_BF16 or DEC_F32.  Rows of other
 * slots are untouched.  Typical step order: dec_kv_append, dec_attn_step,
 * dec_sample_topk(_philox), dec_step_advance. */
int dec_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* len, int n_layers, int B, int H, int L_cap, int hd, int dtype,
                  dec_stream_t stream);

/* The merged 9-codebook LM head on the last position ("Analysis and
 * improvements": logits only for the last position; the nine heads merged into
 * one weight matrix):
 *   logits[b, c, v] = sum_d h[b, d] * W[c, v, d]     for v < V_valid
 *   h       [B, D] bf16              the decoder's last hidden state
 *   W       [n_cb, V_stride, D] bf16 rows v >= V_valid are never read
 *   logits  [B, n_cb, V_stride] fp32 (the dec_sample_topk input); columns
 *           v >= V_valid are left untouched
 * No bias.  fp32 accumulation.  D one of 512, 768, 1024, 1536, 2048, else
 * DEC_E_UNSUPPORTED; (V_valid + 64) * D * 2 below 2^31 bytes; h and W 16-byte
 * aligned, logits 4-byte aligned.  Device pointers, caller-owned.  At B <= 2 the
 * product is a matrix-vector product and runs on the vector ALU; larger batches run
 * on MFMA when logits is 16-byte aligned, V_stride a multiple of 4 and
 * (B + 32) * D * 2 below 2^31 bytes (otherwise on the vector ALU too).  Both kernels
 * read W in whole cache lines in the same order; they round differently but stay
 * within the same fp32 accumulation bound. */
int dec_lm_head(const void* h, const void* W, float* logits, int B, int D, int n_cb,
                int V_valid, int V_stride, dec_stream_t stream);

/* The merged 9-codebook embedding lookup: the decoder input of the next step
 * is the sum of the codebooks' embedding rows ("Analysis and improvements":
 * nine lookups merged into one; "A rough architecture of Parler TTS": all nine
 * tokens of a step enter together):
 *   x[b, d] = sum_c E[c, tokens[b, c], d]   (codebook order, fp32)
 *   tokens [B, n_cb] int32; a token outside [0, V_emb) adds nothing (the fill
 *          token needs a row of its own to contribute)
 *   E      [n_cb, V_emb, D] bf16, 16-byte aligned, D a multiple of 8
 *   x      [B, D] fp32, 16-byte aligned
 * B <= 65535.  Device pointers, caller-owned. */
int dec_embed_sum(const int32_t* tokens, const void* E, float* x, int B, int n_cb, int V_emb,
                  int D, dec_stream_t stream);

/* Advance device-resident decode state by one step inside a captured graph:
 * len[b] += 1 (if len != NULL) and step[b] += 1 (if step != NULL) for b < B. */
int dec_step_advance(int32_t* len, int32_t* step, int B, dec_stream_t stream);

/* The uniforms of a run of decode steps, drawn in one launch ahead of them
 * ("Analysis and improvements": sampling without a GPU/CPU synchronisation; with
 * the random numbers drawn on the device no step needs host input).  A sampler
 * launch then reads its step's uniforms (the `uniforms` argument of
 * dec_sample_topk, _ex or _advance) instead of drawing them in its own launch,
 * where the ten dependent Philox rounds lengthen the row's critical path.
 *   out   [n_steps, B, n_cb] float32, 4-byte aligned (DEC_E_ALIGN): out[s, b, c]
 *         = the uniform of row (b, c) at step step0 + s, exactly the value
 *         dec_sample_topk_philox draws for that row when step[b] = step0 + s
 *         (Philox4x64-10, counter (step0 + s, b, c, 0), key (seed, 0), the top
 *         24 bits of output word 0 times 2^-24)
 * n_steps, B, n_cb >= 1, step0 >= 0, step0 + n_steps and n_steps * B * n_cb
 * below 2^31 (else DEC_E_SHAPE); out NULL: DEC_E_NULL.  Device pointer,
 * caller-owned; nothing else is read or written. */
int dec_philox_uniforms(uint64_t seed, int step0, int n_steps, int B, int n_cb, float* out,
                        dec_stream_t stream);

/* Calibration for the measurements; neither is a step of a decode step.
 * dec_probe_read streams [buf, buf + bytes) once (16-byte non-temporal loads,
 * 8 KiB per wavefront, one workgroup of four wavefronts per 32 KiB), giving
 * the HBM read bandwidth this part reaches for that byte count in one launch:
 * the ceiling an attention launch of the same bytes is compared against,
 * beside the specification peak.  A lane whose 32 words XOR to 0x9E3779B9
 * stores its global lane index (wavefront * 64 + lane, where wavefront w reads
 * bytes [8192 w, 8192 w + 8192) and lane l of it the 16 bytes at 16 l + 1024 u,
 * u = 0..7) to sink[0]; nothing else is written.  buf 16-byte aligned, bytes a
 * positive multiple of 16 (else DEC_E_ALIGN / DEC_E_SHAPE); device pointers,
 * caller-owned.  dec_probe_empty launches one wavefront that does nothing: the
 * fixed cost of one node of a captured graph. */
int dec_probe_read(const void* buf, size_t bytes, uint32_t* sink, dec_stream_t stream);
int dec_probe_empty(dec_stream_t stream);

/* Calibration too: marks a point in a stream or a captured graph.  Launches
 * DEC_PROBE_CLOCK_SLOTS single-wave workgroups; the dispatcher deals them to the
 * XCDs in turn, and each writes its XCD's constant-rate clock (100 MHz, 10 ns per
 * tick) to clocks[XCD id].  clocks: DEC_PROBE_CLOCK_SLOTS uint64 entries, device,
 * 8-byte aligned (else DEC_E_NULL / DEC_E_ALIGN); entries of XCDs that ran no
 * workgroup keep their value.  XCDs keep separate clocks, offset by microseconds:
 * compare a slot only with the same slot of other readings. */
#define DEC_PROBE_CLOCK_SLOTS 16
int dec_probe_clock(uint64_t* clocks, dec_stream_t stream);

/* Graph capture of a whole decode step ("Analysis and improvements": the step
 * is captured once and replayed with a single launch).  begin/end bracket
 * ordinary dec_* calls on a non-default stream; end returns an executable
 * graph in *exec (an opaque hipGraphExec_t). */
int dec_graph_begin(dec_stream_t stream);
int dec_graph_end(dec_stream_t stream, void** exec);
int dec_graph_launch(void* exec, dec_stream_t stream);
int dec_graph_destroy(void* exec);

/* Test and tuning overrides of the launch policy, for the calling thread only (the
 * library keeps no other per-call state).  They change how work is cut and spread,
 * never what is computed: every setting gives results within the same parity bars.
 * The defaults (all fields 0) are what every product call uses; tests use the
 * overrides to reach each schedule and to compare them bit for bit.
 *   attn_chunk_keys  0: the launcher chooses; else keys per split-K chunk, a power of
 *                    two from 128 to 1024 (a call whose workspace does not hold the
 *                    chunk states at that chunk returns DEC_E_UNSUPPORTED)
 *   attn_schedule    0: by call shape; 1: every chunk its own work item; 2: one
 *                    workgroup per sequence (no cross-workgroup fold)
 *   attn_blocks      0: the occupancy-sized persistent grid; else that many workgroups
 *   attn_no_halves   1: whole-sequence launches never cut heavy sequences in halves
 *   attn_no_records  1: launches do not request the tiles recorded by the last launch
 *   head_kernel      0: by shape; 1: the vector-ALU kernel at every batch size; 2: the
 *                    MFMA kernel wherever its alignment allows
 *   head_mfma_cfg    0: the measured policy; else the MFMA kernel's tiling per
 *                    workgroup as 10 * row tiles + batch tiles: 11, 12, 22 or 42
 * dec_tuning_set(NULL) restores the defaults.  Returns DEC_E_SHAPE for a value out of
 * range (nothing is changed). */
typedef struct dec_tuning {
  int attn_chunk_keys;
  int attn_schedule;
  int attn_blocks;
  int attn_no_halves;
  int attn_no_records;
  int head_kernel;
  int head_mfma_cfg;
} dec_tuning;
int dec_tuning_set(const dec_tuning* t);
/* The calling thread's current overrides. */
int dec_tuning_get(dec_tuning* t);

/* The hipError_t of the last failed HIP call made by this thread. */
int dec_last_hip_error(void);

/* A static string naming a dec_status code. */
const char* dec_strerror(int status);

/* Host-only helper: the order-preserving float -> uint32 key map that the
 * sampler's top-k selection uses (a < b  =>  key(a) < key(b); -0 and +0 map
 * alike).  keys[i] = key(x[i]) for i < n.  Both pointers are HOST pointers.
 * Exposed so the map can be checked exhaustively on the CPU. */
void dec_order_keys_host(const float* x, uint32_t* keys, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* DECSTEP_H */
