/*
 * mk_stream.h -- C ABI of the read-bandwidth probe that the benchmark measures the megakernel against.
 *
 * The megakernel's step is bound by HBM bandwidth: every token reads the weights from
 * high-bandwidth memory (news digest "TPU 巨核:同样是 16 块芯片,Kimi K3 快 57%", section
 * 差距从哪里来). This probe reads a buffer once with each of the load kinds the megakernel uses, so
 * that its achieved bandwidth can be stated against a measured read rate of the same machine as well
 * as against the vendor peak, and so that hardware traffic counters can be calibrated per load kind.
 * It is not part of the decode path.
 */
#ifndef MK_STREAM_H
#define MK_STREAM_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MK_STREAM_WEIGHTS = 0,  /* 16-byte non-temporal global loads, as the weight and cache rows are read */
  MK_STREAM_COHERENT = 1, /* 16-byte device-coherent buffer loads, as activations are read */
  MK_STREAM_TO_LDS = 2,   /* 16-byte memory-to-LDS copies, as inputs are staged */
  MK_STREAM_CACHED = 3    /* 16-byte global loads with the default cache policy */
} mk_stream_kind;

/* Read bytes of device memory at d_buf once with the given load kind, asynchronously on hip_stream,
 * and fold what was read into d_sink (device, 4096 uint32 words, written; its contents are
 * meaningless, it only keeps the loads from being removed). d_buf must be 256-byte aligned and
 * bytes a positive multiple of 16 KiB, at most 2^40 (a pass over a buffer that fits the
 * last-level cache, repeated, measures that cache instead of HBM). Returns 0, -1 for a bad argument (NULL
 * pointer, misalignment, bad size or kind), or -5 when the launch fails. */
int mk_stream_read(const void* d_buf, uint64_t bytes, int kind, uint32_t* d_sink, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
