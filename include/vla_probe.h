/* Measurement probes of the policy-step library (libvla.so).
 *
 * Not part of the policy interface (vla.h): these calls time one kernel class
 * of a model's own launches with HIP events, for benchmarks and profiles.  They
 * change no result (except as stated for vla_probe_arm_ex) and cost nothing
 * while no probe is armed.  Same threading and error conventions as vla.h.
 */
#ifndef VLA_PROBE_H_
#define VLA_PROBE_H_

#include "vla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel probes, for measurement.  While a probe is armed on a model, each of
 * the next `max_launches` launches of the chosen kernel class issued by that
 * model outside a HIP graph is bracketed by a pair of HIP events on the stream
 * it runs on.  vla_probe_read synchronises those events and returns the summed
 * device time of the bracketed launches and their count; arming again resets
 * the probe, kind 0 disarms it.  Probes add two event records per launch and
 * nothing else to the measured work. */
typedef enum {
  VLA_PROBE_NONE = 0,
  VLA_PROBE_PREFIX_GATEUP = 1, /* prefix gate/up projection with the GeGLU epilogue */
  VLA_PROBE_PREFIX_DOWN = 2,   /* prefix down projection                            */
  VLA_PROBE_PREFIX_QKV = 3,    /* prefix fused Q/K/V projection                     */
  VLA_PROBE_PREFIX_ATTN = 4,   /* prefix bidirectional attention                    */
  VLA_PROBE_PREFIX_O = 5,      /* prefix output projection                          */
  VLA_PROBE_CACHE = 6,         /* cache-writing projection                          */
  VLA_PROBE_EXPERT_SELF_ATTN = 7,  /* action-expert self (or joint) attention          */
  VLA_PROBE_EXPERT_CROSS_ATTN = 8, /* action-expert cross-attention into the cache     */
  VLA_PROBE_EXPERT_SCORES = 9,     /* absorbed cross sublayer: the score product        */
  VLA_PROBE_EXPERT_GATEUP = 10     /* action-expert gate/up projection with the GeGLU   */
} vla_probe_kind;
vla_status vla_probe_arm(vla_model* model, int32_t kind, int32_t max_launches);
/* The same with each bracketed launch issued `repeat` (1..1000) times back to
 * back between its two events, so the events' own cost is spread over many
 * launches; vla_probe_read then counts every repeat as a launch.  A kernel
 * that adds into its output (a residual update) adds `repeat` times: the
 * results of calls made while such a probe is armed are for timing only. */
vla_status vla_probe_arm_ex(vla_model* model, int32_t kind, int32_t max_launches, int32_t repeat);
vla_status vla_probe_read(vla_model* model, float* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* VLA_PROBE_H_ */
