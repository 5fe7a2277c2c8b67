/*
 * avae.h -- C-ABI of libavae.so: the alias-free BigVGAN waveform decoder on
 * one MI355X (gfx950).
 *
 * Sources of the operations (cited by page and item):
 *   [H3]  docs.rs source page of cortiq_engine/audiovae.rs (cortiq-engine
 *         0.5.74): the MiniMax-H3 audio VAE decoder.
 *   [LTX] docs.rs source page of cortiq_engine/ltxaudio.rs (cortiq-engine
 *         0.6.3): the LTX-2.5 BigVGAN v2 vocoder.
 *
 * Conventions for every entry point
 *   - Tensors are float32, contiguous, row-major, in DEVICE memory unless a
 *     parameter says "host".  Activations are [B, C, T]: B independent mono
 *     passes (stereo = B 2), C channels, T samples, time fastest.
 *   - The caller owns every buffer it passes; the library never frees or
 *     keeps a caller pointer beyond the call, except that a decoder keeps
 *     its own copy of the weights (avae_decoder_create).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every compute
 *     call is asynchronous on that stream, allocates nothing and never
 *     synchronises.
 *   - Return value: AVAE_OK (0) on success, or a negative AVAE_E* code.
 *     All argument and shape checks happen before anything is launched, so
 *     a failed call has no effect on the device.  avae_last_error() gives a
 *     message for the last failure on the calling thread.
 *   - Input and output buffers must not overlap unless a parameter says so.
 */
#ifndef AVAE_H
#define AVAE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AVAE_OK          0
#define AVAE_EINVAL     -1 /* null pointer, non-positive size, bad enum      */
#define AVAE_ESHAPE     -2 /* shapes that do not fit together or exceed a cap */
#define AVAE_EWORKSPACE -3 /* workspace missing or too small                 */
#define AVAE_EHIP       -4 /* the HIP runtime reported an error               */
#define AVAE_ENOMEM     -5 /* device allocation failed (create only)          */

#define AVAE_FILTER_LEN   12 /* [H3] FILTER_LEN: both resampling filters       */
#define AVAE_MAX_STAGES    8
#define AVAE_MAX_KERNELS   4
#define AVAE_MAX_DIL       4
#define AVAE_MAX_TAPS     31 /* largest Conv1d / ConvTranspose1d kernel size  */

enum avae_final { AVAE_FINAL_NONE = 0, AVAE_FINAL_TANH = 1, AVAE_FINAL_CLAMP = 2 };

/* Message for the last non-zero return on this thread ("" if none). */
const char* avae_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int avae_version(void);

/*
 * Kaiser-windowed sinc lowpass taps, designed in float64 on the host and
 * rounded to float32, normalised to unit sum ([H3] kaiser_sinc, bessel_i0,
 * sinc).  Tap i sits at t = i - taps/2 + 0.5; window I0(beta*sqrt(1-r^2))/I0(beta)
 * with r = 2i/(taps-1) - 1 and Kaiser's beta for the attenuation
 * 2.285*(taps/2 - 1)*pi*(4*half_width) + 7.95.  The decoder's filters are
 * avae_kaiser_sinc(0.25, 0.3, 12, out).
 *   out_host: host array of `taps` floats (written).
 * Errors: EINVAL for taps < 2, taps odd, cutoff or half_width not in (0, 0.5].
 * Touches no device.
 */
int avae_kaiser_sinc(double cutoff, double half_width, int taps, float* out_host);

/*
 * Alias-free activation, [B, C, T] -> [B, C, T] ([H3] Activation1d::apply,
 * SnakeBeta, fir_pad; [LTX] Aliasing::upsample/downsample, SnakeBeta::forward):
 *   mid = x2 upsample: replicate-pad 5 each side, transposed FIR (stride 2,
 *         gain 2) with up_taps, trim 15 each side  -> 2T samples;
 *   mid = mid + sin^2(exp(log_alpha[c]) * mid) / (exp(log_beta[c]) + 1e-9);
 *   y   = replicate-pad mid 5 left / 6 right, FIR with down_taps, stride 2.
 *   x, y:                 [B, C, T] device; must not overlap.
 *   log_alpha, log_beta:  [C] device, log-scale SnakeBeta parameters.
 *   up_taps, down_taps:   HOST arrays of AVAE_FILTER_LEN floats, or NULL for
 *                         the designed avae_kaiser_sinc(0.25, 0.3, 12) taps.
 * Errors: EINVAL (null tensor, B, C or T < 1).
 */
int avae_act1d(const float* x, float* y, int B, int C, int T,
               const float* log_alpha, const float* log_beta,
               const float* up_taps, const float* down_taps, void* stream);

/*
 * Dilated Conv1d with zero padding ([H3] Conv1d::apply, get_padding):
 *   y[b,o,t] = bias[o] + sum_i sum_j w[o,i,j] * x[b,i, t + j*dilation - pad]
 *              (+ residual[b,o,t] if residual != NULL)
 *   Tout = T + 2*pad - dilation*(K-1)  (the "same" length for pad = (K*d-d)/2).
 *   x: [B, Cin, T]; y: [B, Cout, Tout]; w: [Cout, Cin, K] (PyTorch layout);
 *   bias: [Cout] or NULL; residual: [B, Cout, Tout] or NULL, and it MAY be
 *   the same buffer as y (in-place residual add, as in [H3] AmpBlock::apply).
 *   Arithmetic: float32 products accumulated in float32 on the FP32 matrix
 *   cores.
 * Errors: EINVAL (null x/y/w, sizes < 1, dilation < 1, pad < 0);
 *         ESHAPE (Tout < 1, K > AVAE_MAX_TAPS).
 */
int avae_conv1d(const float* x, float* y, int B, int Cin, int Cout, int T,
                const float* w, const float* bias, int K, int dilation, int pad,
                const float* residual, void* stream);

/*
 * The same "same"-padded Conv1d (pad = (K-1)*dilation/2, Tout = T) through
 * the convolution theorem ([H3] Conv1d::apply; overlap-save framing):
 * each row is cut into blocks of L = 256 - (K-1)*dilation outputs, every
 * block's 256-sample input window is transformed, the channels are mixed
 * by one complex matrix product per frequency on the FP32 matrix cores,
 * and the L valid samples of each block's inverse transform are kept.
 * Same result as avae_conv1d up to float32 rounding (a few 1e-6 of the
 * output's RMS).  Takes Cin and Cout multiples of 16, odd K and
 * (K-1)*dilation <= 128.
 *
 * avae_conv1d_fft_weight_floats: floats of the packed weights for (Cin, Cout).
 * avae_conv1d_fft_pack: w [Cout, Cin, K] (device) -> wp (device, that many
 *   floats, caller-owned): the frequency responses of every (o, i) filter at
 *   the given dilation, summed in double and rounded to float32, in the
 *   matrix kernel's operand order.  Pack once per weight tensor and dilation.
 * avae_conv1d_fft_workspace_bytes: device workspace avae_conv1d_fft needs
 *   (the two spectra); 0 if the shape is not supported.
 * avae_conv1d_fft: x [B, Cin, T], y [B, Cout, T] (must not overlap x or the
 *   workspace), wp from avae_conv1d_fft_pack with the same K and dilation,
 *   bias [Cout] or NULL, residual [B, Cout, T] or NULL (may be y).
 * Errors: EINVAL (null pointers, sizes < 1, x == y); ESHAPE (unsupported
 *   Cin, Cout, K or dilation); EWORKSPACE (workspace too small).
 */
size_t avae_conv1d_fft_weight_floats(int Cin, int Cout);
int avae_conv1d_fft_pack(const float* w, float* wp, int Cin, int Cout, int K, int dilation,
                         void* stream);
size_t avae_conv1d_fft_workspace_bytes(int B, int Cin, int Cout, int T, int K, int dilation);
int avae_conv1d_fft(const float* x, float* y, int B, int Cin, int Cout, int T, const float* wp,
                    const float* bias, int K, int dilation, const float* residual,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * avae_conv1d_fft of Activation1d(x): the activation of an AMP block's
 * act -> conv pair ([H3] AmpBlock::apply, Activation1d::apply) with the
 * designed avae_kaiser_sinc(0.25, 0.3, 12) taps, evaluated on each block's
 * window inside the forward transforms (the activation never goes to
 * memory).  Arguments as avae_conv1d_fft, plus log_alpha, log_beta [Cin]
 * (device) as in avae_act1d.  Same result as avae_act1d followed by
 * avae_conv1d_fft up to float32 rounding.
 */
int avae_act_conv1d_fft(const float* x, float* y, int B, int Cin, int Cout, int T,
                        const float* log_alpha, const float* log_beta, const float* wp,
                        const float* bias, int K, int dilation, const float* residual,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * ConvTranspose1d ([H3] ConvT1d::apply/load; [LTX] ConvT1d):
 *   y[b, o, t*stride + j - pad] += x[b,i,t] * w[i,o,j], plus bias[o];
 *   Tout = (Tin - 1)*stride + K - 2*pad.
 *   Computed as `stride` polyphase gathers (no atomics, no zero-stuffing).
 *   x: [B, Cin, Tin]; y: [B, Cout, Tout]; w: [Cin, Cout, K] (PyTorch layout);
 *   bias: [Cout] or NULL; pad < 0 selects (K - stride)/2 (integer division,
 *   the pages' choice; needs K >= stride).
 * Errors: EINVAL (null x/y/w, sizes < 1, stride < 1);
 *         ESHAPE (Tout < 1, K > AVAE_MAX_TAPS, pad < 0 with K < stride).
 */
int avae_convtr1d(const float* x, float* y, int B, int Cin, int Cout, int Tin,
                  const float* w, const float* bias, int K, int stride, int pad,
                  void* stream);

/*
 * One AMP residual block ([H3] AmpBlock::apply, [LTX] AmpBlock::forward):
 *   cur = x; for q < n_dil:
 *     cur += conv2_q(act_{2q+1}(conv1_q(act_{2q}(cur))))
 *   with conv1_q of kernel K, dilation dil[q], "same" padding, and conv2_q of
 *   kernel K, dilation 1.  Then
 *     y = out_scale * cur            (accumulate == 0)
 *     y = y + out_scale * cur        (accumulate != 0)
 *   which gives the MRF average of [H3] AudioVae::decode with
 *   out_scale = 1/n_kernels over n_kernels calls into one y.
 *   x, y: [B, C, T] device, must not overlap.
 *   dil: HOST array [n_dil].  w1, b1, w2, b2: HOST arrays [n_dil] of device
 *   pointers (w: [C, C, K]; b: [C] or NULL).  log_alpha, log_beta: HOST
 *   arrays [2*n_dil] of device pointers to [C] (activation q's parameters).
 *   Activations use the designed taps.
 *   workspace: device, at least avae_amp_block_workspace_bytes(B, C, T).
 *   With at least avae_amp_block_fft_workspace_bytes(B, C, T, K, n_dil, dil)
 *   bytes (larger for the shapes that take it), the block's convolutions
 *   whose width and taps suit the 256-point overlap-save form (as in
 *   avae_conv1d_fft, with the activation inside its forward transforms) run
 *   that way, their weights packed into the workspace on each call; the
 *   result is the same up to float32 rounding.
 * Errors: EINVAL, ESHAPE (n_dil > AVAE_MAX_DIL, K even or > AVAE_MAX_TAPS),
 *         EWORKSPACE.
 */
size_t avae_amp_block_workspace_bytes(int B, int C, int T);
/* Workspace bytes that select the frequency-domain path (equal to
 * avae_amp_block_workspace_bytes(B, C, T) where no convolution takes it);
 * 0 for invalid arguments (n_dil outside [1, AVAE_MAX_DIL], null dil). */
size_t avae_amp_block_fft_workspace_bytes(int B, int C, int T, int K, int n_dil,
                                          const int* dil);
int avae_amp_block(const float* x, float* y, int B, int C, int T, int K,
                   int n_dil, const int* dil,
                   const float* const* w1, const float* const* b1,
                   const float* const* w2, const float* const* b2,
                   const float* const* log_alpha, const float* const* log_beta,
                   float out_scale, int accumulate,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * avae_amp_block for callers that cannot allocate device memory (code under
 * stream/graph capture, tight serving loops, hosts that forbid hipMalloc):
 * the same computation, arguments and results as avae_amp_block, without
 * the workspace arguments.  Its scratch (the three [B, C, T] slots and the
 * packed weights of avae_amp_block's workspace) is a static device array
 * of AVAE_AMP_STATIC_SCRATCH_MB MiB built into the library: each GPU the
 * library runs on holds its own copy from the library's load until the
 * process ends.  The call allocates nothing (no hipMalloc, no hipFree) and
 * never synchronises; its device address is looked up on the first call on
 * each device.
 *   Limit: avae_amp_block_workspace_bytes(B, C, T) must not exceed
 *   avae_amp_block_static_max_bytes() (ESHAPE otherwise), e.g. B*C*T up to
 *   about 5.5 M samples at C > 24.
 *   Concurrency: every call on one GPU shares that GPU's array, which keeps
 *   the last call's contents; two calls that overlap on one GPU (on
 *   different streams, or from different host threads without ordering
 *   between their streams) race and give wrong results.  Calls ordered on
 *   one stream are safe.
 * Errors: as avae_amp_block, with ESHAPE for sizes over the limit instead
 * of EWORKSPACE, and EHIP if the scratch address cannot be looked up.
 */
#define AVAE_AMP_STATIC_SCRATCH_MB 64
size_t avae_amp_block_static_max_bytes(void);
int avae_amp_block_static(const float* x, float* y, int B, int C, int T, int K,
                          int n_dil, const int* dil,
                          const float* const* w1, const float* const* b1,
                          const float* const* w2, const float* const* b2,
                          const float* const* log_alpha, const float* const* log_beta,
                          float out_scale, int accumulate, void* stream);

/*
 * Whole decoder ([H3] AudioVae::from_cmf/decode; [LTX] Vocoder::forward):
 *   [optional z*std + mean] -> [optional 1x1 dec_in conv] -> conv_pre
 *   (k_pre, "same") -> per stage i: ConvTranspose1d (rate rates[i], kernel
 *   up_k[i], pad (up_k[i]-rates[i])/2) then the MRF average of n_kernels AMP
 *   blocks -> act_post -> conv_post (k_post, "same", 1 channel) -> final
 *   (none / tanh / clamp to [-1, 1]).
 *   Channel widths: ch[0] = conv_pre output, ch[i+1] = stage i output.
 */
typedef struct avae_config {
    int c_in;                       /* latent channels                          */
    int dec_in_ch;                  /* >0: 1x1 dec_in conv c_in -> dec_in_ch     */
    int has_latent_affine;          /* !=0: z*latent_std + latent_mean first     */
    int k_pre, k_post;              /* conv_pre / conv_post kernel sizes (odd)   */
    int n_stages;
    int ch[AVAE_MAX_STAGES + 1];
    int rates[AVAE_MAX_STAGES];
    int up_k[AVAE_MAX_STAGES];
    int n_kernels;                  /* AMP blocks per stage                      */
    int rb_k[AVAE_MAX_KERNELS];     /* their kernel sizes (odd)                  */
    int n_dil;                      /* dilations per AMP block                   */
    int rb_d[AVAE_MAX_KERNELS][AVAE_MAX_DIL];
    int final_act;                  /* enum avae_final                           */
} avae_config;

/* Device pointers to the caller's weights (PyTorch layouts).  Biases may be
 * NULL (treated as zero).  Unused entries are ignored. */
typedef struct avae_weights {
    const float* latent_mean;       /* [c_in]                                   */
    const float* latent_std;        /* [c_in]                                   */
    const float* dec_in_w;          /* [dec_in_ch, c_in, 1]                     */
    const float* dec_in_b;
    const float* conv_pre_w;        /* [ch0, c_in or dec_in_ch, k_pre]          */
    const float* conv_pre_b;
    const float* up_w[AVAE_MAX_STAGES];   /* [ch[i], ch[i+1], up_k[i]]          */
    const float* up_b[AVAE_MAX_STAGES];
    const float* w1[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][AVAE_MAX_DIL]; /* [C,C,k] */
    const float* b1[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][AVAE_MAX_DIL];
    const float* w2[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][AVAE_MAX_DIL];
    const float* b2[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][AVAE_MAX_DIL];
    const float* act_la[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][2 * AVAE_MAX_DIL];
    const float* act_lb[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][2 * AVAE_MAX_DIL];
    const float* post_la;           /* [ch[n_stages]]                           */
    const float* post_lb;
    const float* conv_post_w;       /* [1, ch[n_stages], k_post]                */
    const float* conv_post_b;       /* [1]                                      */
} avae_weights;

typedef struct avae_decoder avae_decoder;

/* Validates the config and copies every weight into one library-owned
 * device allocation on the current device (synchronous; the only call that
 * allocates).  *out receives the decoder.  Errors: EINVAL, ESHAPE, ENOMEM,
 * EHIP. */
int avae_decoder_create(const avae_config* cfg, const avae_weights* w, avae_decoder** out);
void avae_decoder_destroy(avae_decoder* dec);

/* Output samples per pass for `frames` latent frames (frames*hop for the
 * pages' kernel/rate pairs).  Errors: EINVAL, ESHAPE. */
int avae_decoder_output_length(const avae_decoder* dec, int frames, int* out_len);

/* Workspace bytes avae_bigvgan_decode needs for B passes of `frames` frames
 * (0 on invalid arguments).  The figure does not depend on the concurrency
 * setting below. */
size_t avae_decoder_workspace_bytes(const avae_decoder* dec, int B, int frames);

/*
 * The AMP blocks of one multi-receptive-field stage ([H3] AudioVae::decode:
 * the stage's AmpBlock outputs are summed, then scaled by 1/n_kernels) all
 * read the same upsampled input and are independent of each other.  With `on` (the default when the config has
 * more than one kernel size), blocks 1.. are enqueued on side streams the
 * decoder owns, forked from the caller's stream after the upsampling and
 * joined back to it (events) before their sum, so their kernels overlap on
 * the GPU; with `on` = 0 every block runs on the caller's stream, one after
 * the other.  The two settings add the blocks in the same order but round
 * the sum differently (the serial schedule accumulates in each block's last
 * convolution epilogue; the overlapped one writes each block's scaled
 * output and adds them in one kernel): about one float32 rounding of each
 * stage's output, which the following stages carry forward with the
 * network's gain (measured on a 128-wide H3-shaped decoder: 4.4e-7 of RMS
 * after the first stage, 2.2e-4 at conv_post).  Takes effect for calls
 * made after it returns; not to be called while another host thread decodes
 * with this decoder.  Errors: EINVAL (null decoder, or `on` with a single
 * kernel size or side streams that could not be created).
 */
int avae_decoder_set_concurrent(avae_decoder* dec, int on);

/*
 * Decode: latent [B, c_in, frames] -> wave [B, L] float32, L from
 * avae_decoder_output_length; each row is an independent mono pass.
 * Concurrent calls on different streams are safe with separate workspaces
 * (the weights are read-only here; the enqueue of a stage's concurrent AMP
 * blocks on the decoder's side streams is serialized by a host mutex).
 * Errors: EINVAL, ESHAPE, EWORKSPACE, EHIP.
 */
int avae_bigvgan_decode(const avae_decoder* dec, const float* latent, int B, int frames,
                        float* wave, void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode and also copy intermediate results out, for stage-by-stage
 * comparison ([H3] AudioVae::decode prints them under CMF_AVAE_PROF).
 * stage_out: HOST array of n_stages + 2 device pointers (any may be NULL):
 *   [0]            conv_pre output     [B, ch[0], frames]
 *   [1 + i]        stage i output      [B, ch[i+1], T_{i+1}]
 *   [n_stages + 1] conv_post output before the final nonlinearity [B, L]
 */
int avae_bigvgan_decode_traced(const avae_decoder* dec, const float* latent, int B, int frames,
                               float* wave, void* workspace, size_t ws_bytes,
                               float* const* stage_out, void* stream);

/*
 * Time-tiled (streaming) decode for long latents.  The latent is decoded in
 * tiles of `tile_frames` frames; each tile is decoded from a crop with
 * `halo_frames` frames of context on every side that is not a sequence end
 * (the first and last tiles: tile_frames + halo_frames frames at their end
 * of the sequence; inner tiles: tile_frames + 2 halo_frames around them;
 * clipped to the sequence) and only the tile's own samples are kept.  Tiles
 * whose crops have the same length are stacked along the batch axis, up to
 * four per decode pass.  The decoder is a
 * finite, non-causal stack of convolutions and resampling filters ([H3]
 * AudioVae::decode), so with halo_frames >= avae_decoder_reach_frames()
 * every kept sample depends only on latent frames inside its crop and
 * equals the whole-sequence decode up to float32 summation order (tile
 * shapes may select different kernel tilings).  The workspace covers four
 * tiles, whatever `frames` is.
 * Requires an exact hop geometry: output length frames * prod(rates)
 * (ESHAPE otherwise).  halo_frames < 0 selects avae_decoder_reach_frames().
 */
int avae_decoder_reach_frames(const avae_decoder* dec, int* out_frames);
size_t avae_decoder_streaming_workspace_bytes(const avae_decoder* dec, int B, int tile_frames,
                                              int halo_frames);
int avae_bigvgan_decode_streaming(const avae_decoder* dec, const float* latent, int B,
                                  int frames, float* wave, int tile_frames, int halo_frames,
                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * Plain Snake ([H3] Snake::apply, the Music-3 DAV decoder's activation):
 * y[b,c,t] = x + sin^2(alpha[c] x) / (alpha[c] + 1e-9), alpha [C] used as
 * stored (no exponential, unlike the SnakeBeta of avae_act1d).  x, y
 * [B, C, T]; y may equal x (pointwise, in place).  EINVAL on null pointers
 * or sizes < 1.
 */
int avae_snake(const float* x, float* y, int B, int C, int T, const float* alpha, void* stream);

/*
 * The MiniMax-Music-3 DAV decoder ([H3] page, items Music3Dav, DavStage,
 * DavUnit, Snake).  Per stereo side (a mono pass): dec_in (1-tap conv,
 * c_side -> dec_in_ch), conv_pre (k_pre taps, "same", -> ch[0]), then per
 * stage i: Snake(stage_alpha[i]) -> ConvTranspose1d (ch[i] -> ch[i+1],
 * stride strides[i], up_k[i] taps, padding (up_k - stride)/2) -> n_units
 * residual units u: x + c2(Snake(c1(Snake(x, a1)), a2)) with c1 unit_k taps
 * at dilation unit_dil[u] ("same") and c2 one tap; then Snake(post_alpha),
 * conv_post (k_post taps, "same", -> 1 channel) and tanh.
 * Weight layouts: Conv1d [Cout, Cin, k], ConvTranspose1d [Cin, Cout, k],
 * biases [Cout] (may be NULL), alphas [C].  Like avae_decoder, the decoder
 * keeps a device copy of the weights (host or device pointers accepted).
 */
typedef struct avae_dav_config {
    int c_side;                      /* latent channels per side (latent has 2 c_side) */
    int dec_in_ch;
    int k_pre, k_post;               /* odd, <= AVAE_MAX_TAPS */
    int n_stages;                    /* <= AVAE_MAX_STAGES */
    int ch[AVAE_MAX_STAGES + 1];
    int strides[AVAE_MAX_STAGES];
    int up_k[AVAE_MAX_STAGES];       /* >= stride */
    int unit_k;                      /* odd */
    int n_units;                     /* <= AVAE_MAX_DIL */
    int unit_dil[AVAE_MAX_DIL];
} avae_dav_config;

typedef struct avae_dav_weights {
    const float *dec_in_w, *dec_in_b;
    const float *conv_pre_w, *conv_pre_b;
    const float *stage_alpha[AVAE_MAX_STAGES];
    const float *up_w[AVAE_MAX_STAGES], *up_b[AVAE_MAX_STAGES];
    const float *a1[AVAE_MAX_STAGES][AVAE_MAX_DIL], *w1[AVAE_MAX_STAGES][AVAE_MAX_DIL],
        *b1[AVAE_MAX_STAGES][AVAE_MAX_DIL];
    const float *a2[AVAE_MAX_STAGES][AVAE_MAX_DIL], *w2[AVAE_MAX_STAGES][AVAE_MAX_DIL],
        *b2[AVAE_MAX_STAGES][AVAE_MAX_DIL];
    const float *post_alpha, *conv_post_w, *conv_post_b;
} avae_dav_weights;

typedef struct avae_dav avae_dav;

/* EINVAL (null, missing weight, bad size), ESHAPE (caps), ENOMEM, EHIP. */
int avae_dav_create(const avae_dav_config* cfg, const avae_dav_weights* w, avae_dav** out);
void avae_dav_destroy(avae_dav* dav);
/* Samples per side for `frames` latent frames (frames * prod(strides) when
 * up_k = 2 stride). */
int avae_dav_output_length(const avae_dav* dav, int frames, int* out_len);
size_t avae_dav_workspace_bytes(const avae_dav* dav, int B, int frames);
/*
 * latent [B, 2 c_side, frames] (channels [0, c_side) the left side, the rest
 * the right: [H3] Music3Dav::decode folds the 2 c_side latent into two mono
 * passes) -> wave [B, 2 L], interleaved: wave[b][2 t + side].  The two sides
 * of all B items run as one batch of 2 B passes.  EWORKSPACE if ws_bytes <
 * avae_dav_workspace_bytes().
 */
int avae_dav_decode(const avae_dav* dav, const float* latent, int B, int frames, float* wave,
                    void* workspace, size_t ws_bytes, void* stream);
/*
 * Same, and copies intermediate results of the [2 B, ...] side batch (row
 * 2 b + side) into stage_out[0 .. n_stages+1] where non-NULL: [0] conv_pre
 * output [2B, ch[0], frames], [1+i] stage i output, [n_stages+1] the
 * conv_post output before tanh [2B, L].
 */
int avae_dav_decode_traced(const avae_dav* dav, const float* latent, int B, int frames,
                           float* wave, void* workspace, size_t ws_bytes,
                           float* const* stage_out, void* stream);

/*
 * LTX bandwidth-extension tail ([LTX] page, items MelStft, hann_sinc_upsample,
 * AudioStack::decode_from_mel).
 *
 * avae_mel_stft: causal log-mel of x [B, T] -> out [B, n_mels, frames] with
 * frames = floor(T / hop): frame f is the STFT (as a product with
 * forward_basis [2 n_freqs, filter_len]: rows r real, rows n_freqs + r
 * imaginary) of samples [f hop - (filter_len - hop), f hop + hop) of x, zero
 * outside [0, T); then sqrt(re^2 + im^2), the mel projection mel_basis
 * [n_mels, n_freqs] and ln(max(., 1e-5)).  Needs filter_len >= hop,
 * filter_len % 32 == 0, n_freqs <= 384 (ESHAPE).  Device pointers.
 *
 * avae_hann_sinc_upsample: y [B, ratio T] = the x`ratio` Hann-windowed sinc
 * interpolation of x [B, T] (rolloff 0.99, 6 zero crossings: 2 w ratio + 1
 * taps with w = 7, designed on the host in float64), replicate-padded at
 * both ends.  ratio in [1, 4].
 *
 * avae_bwe_*: the whole tail.  The 16 kHz signal low [B, T] is zero-padded to
 * Tp = ceil(T / hop) hop samples, its log-mel (Tp / hop frames) drives the
 * extension generator (a BigVGAN decoder, cfg.gen / w.gen exactly as for
 * avae_decoder_create, whose hop prod(rates) must equal hop * ratio and whose
 * final_act is the caller's: the [LTX] page adds its output as a residual),
 * and out [B, ratio T] = clamp(residual + hann_sinc_upsample(padded), -1, 1).
 * avae_bwe_decode_traced also copies the log-mel [B, n_mels, Tp / hop] and
 * the residual [B, Tp * ratio] where non-NULL.
 */
int avae_mel_stft(const float* x, float* out, int B, int T, const float* forward_basis,
                  int n_freqs, int filter_len, int hop, const float* mel_basis, int n_mels,
                  void* stream);
int avae_hann_sinc_upsample(const float* x, float* y, int B, int T, int ratio, void* stream);

typedef struct avae_bwe_config {
    avae_config gen;
    int filter_len, hop, n_freqs, n_mels, ratio;
} avae_bwe_config;

typedef struct avae_bwe_weights {
    avae_weights gen;
    const float *forward_basis, *mel_basis;
} avae_bwe_weights;

typedef struct avae_bwe avae_bwe;

int avae_bwe_create(const avae_bwe_config* cfg, const avae_bwe_weights* w, avae_bwe** out);
void avae_bwe_destroy(avae_bwe* bwe);
size_t avae_bwe_workspace_bytes(const avae_bwe* bwe, int B, int T);
int avae_bwe_decode(const avae_bwe* bwe, const float* low, int B, int T, float* out,
                    void* workspace, size_t ws_bytes, void* stream);
int avae_bwe_decode_traced(const avae_bwe* bwe, const float* low, int B, int T, float* out,
                           void* workspace, size_t ws_bytes, float* mel_out, float* resid_out,
                           void* stream);

/*
 * Launch profiler, the device-side counterpart of the audio decoder's own
 * phase report ([H3] AVAE_TIME / avae_time_report, phases dec_in, conv_pre,
 * upsamples, resblocks, act_post, conv_post).  Between avae_profile_begin and
 * avae_profile_end every kernel launched by this library (any entry point,
 * any stream) is bracketed by two hipEvents and tagged with its kernel name,
 * its decode phase and its algorithmic flops and bytes.  The events are
 * created by avae_profile_begin (room for max_launches launches), so compute
 * calls inside the region still allocate nothing.  Process-wide: one region
 * at a time, driven from one host thread.
 *   avae_profile_begin: EINVAL (max_launches < 1), EHIP.
 *   avae_profile_end:   synchronises on the last event and aggregates per
 *                       kernel name; ESHAPE if launches were dropped because
 *                       the region overflowed max_launches.
 *   avae_profile_entry: entry i < avae_profile_count(): name (copied into
 *                       `name`, NUL-terminated), launches, summed event time
 *                       in ms, summed algorithmic flops and bytes.
 *   avae_profile_phases: host array of 6 doubles, ms per decode phase.
 */
int avae_profile_begin(int max_launches);
int avae_profile_end(void);
int avae_profile_count(void);
int avae_profile_entry(int i, char* name, int name_len, long long* launches, double* total_ms,
                       double* flops, double* bytes);
int avae_profile_phases(double* ms6);

/*
 * Matrix-core throughput probe, a measurement aid for the convolutions'
 * roofline (not part of any decode).  Launches `blocks` workgroups of 256
 * threads on `stream`; every wave runs `chains` (8 or 16) independent
 * v_mfma_f32_16x16x4_f32 accumulator chains for `iters` iterations with no
 * memory traffic in the loop: blocks * 4 * iters * chains * 2048 flops.
 * `sink` is a device buffer of blocks * 256 floats that receives the sums
 * (so the work is kept).  The caller times it (hipEvents on `stream`);
 * with 256 * n blocks each SIMD holds n waves.  Errors: EINVAL (null sink,
 * chains not 8 or 16, blocks or iters < 1), EHIP.
 */
int avae_probe_mfma(int chains, int blocks, int iters, float* sink, void* stream);

/*
 * Streaming-copy probe, a measurement aid for the HBM roofline of the
 * memory-bound kernels (Activation1d): y[i] = x[i] for i < n, one float4 per
 * thread, enqueued on `stream` (the caller times it: 8 n bytes moved).
 * x and y are device buffers of n floats, 16-byte aligned, not overlapping.
 * Errors: EINVAL (null pointer, n not a positive multiple of 4, misaligned
 * buffers), EHIP.
 */
int avae_probe_copy(const float* x, float* y, long long n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AVAE_H */
