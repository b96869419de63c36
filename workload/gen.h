/* Seeded synthetic inputs shared by the CPU oracle and the GPU path.
 * No method arithmetic lives here: only draws and the Q4_0 encoding of drawn
 * weights (the GGUF block format both sides consume). */
#ifndef WORKLOAD_GEN_H
#define WORKLOAD_GEN_H
#include <stdint.h>
#include <stdlib.h>

#define WL_FMT_F32 0
#define WL_FMT_Q4_0 1

#ifdef __cplusplus
extern "C" {
#endif

void wl_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);
void wl_normal_f32(uint64_t seed, uint64_t tensor, uint64_t a, uint64_t b, int64_t n, float sigma,
                   float* out);
double wl_uniform(uint64_t seed, uint64_t tensor, uint64_t a, uint64_t b, uint64_t i);
uint16_t wl_f32_to_f16(float f);
float wl_f16_to_f32(uint16_t h);
void wl_q4_0_encode_block(const float* w, uint8_t* out);
void wl_q4_0_encode(int64_t rows, int64_t cols, const float* w, uint8_t* out);
void wl_router(uint64_t seed, int layer, int E, int d, float sigma, float* wr);
int64_t wl_matrix_bytes(int rows, int cols, int wfmt);
int wl_expert(uint64_t seed, int layer, int expert, int d, int f, int wfmt, float sigma, void* gate,
              void* up, void* down, float* scratch);
int wl_experts(uint64_t seed, int layer0, int n_layers, int E, int d, int f, int wfmt, float sigma,
               uint8_t* out);
void wl_tokens(uint64_t seed, uint64_t stream, int64_t t0, int64_t T, int d, float* x);
void wl_zipf_bias(uint64_t seed, int layer, int E, double alpha, double scale, float* bias,
                  int32_t* rank_out);

#ifdef __cplusplus
}
#endif
#endif
