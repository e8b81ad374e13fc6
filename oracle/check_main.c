/*
 * Driver for the sanitizer build of the oracle (AddressSanitizer, UndefinedBehaviorSanitizer):
 * every oracle routine, both precisions, on small shapes that span the edge cases (one step,
 * one unit, several layers, rows of zero length), plus the rejected arguments. TEST
 * INFRASTRUCTURE ONLY, like the oracle itself. Exit status 0 when every call returned what it
 * should and every output is finite.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_projection_f64(long rows, int in, int hidden, const float *x, const double *x_real, const float *w,
                          const float *b, double *out);
int oracle_projection_f32(long rows, int in, int hidden, const float *x, const float *x_real, const float *w,
                          const float *b, float *out);
int oracle_recurrence_f64(int steps, int hidden, const double *gates, const float *r, double *y);
int oracle_recurrence_f32(int steps, int hidden, const float *gates, const float *r, float *y);
int oracle_stack_window_f64(int steps, int in0, int hidden, int layers, const float *x, const float *w_all,
                            const float *r_all, const float *b_all, double *y, double *gates_dump);
int oracle_stack_window_f32(int steps, int in0, int hidden, int layers, const float *x, const float *w_all,
                            const float *r_all, const float *b_all, float *y, float *gates_dump);
int oracle_heads_f64(long rows, int in, int mid0, int mid1, int classes, double slope, const float *y,
                     const double *y_real, const float *w0, const float *b0, const float *w1, const float *b1,
                     const float *w2, const float *b2, double *out);

static unsigned state = 7u;
static float rnd(void) {
    state = state * 1664525u + 1013904223u;
    return (float)(state >> 8) / 16777216.0f - 0.5f;
}
static float *rand_array(size_t n) {
    float *a = malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) a[i] = rnd();
    return a;
}

static int failures = 0;
static void expect(int ok, const char *what) {
    if (!ok) {
        printf("FAIL %s\n", what);
        ++failures;
    }
}
static int finite_d(const double *a, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

int main(void) {
    const int shapes[][4] = {{1, 1, 1, 1}, {3, 2, 4, 2}, {5, 60, 8, 4}, {2, 7, 3, 3}, {9, 16, 16, 4}};
    for (size_t c = 0; c < sizeof(shapes) / sizeof(shapes[0]); ++c) {
        const int steps = shapes[c][0], in0 = shapes[c][1], hidden = shapes[c][2], layers = shapes[c][3];
        const int g = 4 * hidden, width = 2 * hidden;
        size_t wn = 0;
        for (int l = 0; l < layers; ++l) wn += (size_t)2 * g * (l == 0 ? in0 : width);
        float *x = rand_array((size_t)steps * in0), *w = rand_array(wn);
        float *r = rand_array((size_t)layers * 2 * g * hidden), *b = rand_array((size_t)layers * 4 * g);
        double *y = malloc(sizeof(double) * steps * width), *dump = malloc(sizeof(double) * layers * steps * 2 * g);
        float *yf = malloc(sizeof(float) * steps * width);
        expect(oracle_stack_window_f64(steps, in0, hidden, layers, x, w, r, b, y, dump) == 0, "stack f64");
        expect(finite_d(y, (size_t)steps * width), "stack f64 finite");
        expect(oracle_stack_window_f64(steps, in0, hidden, layers, x, w, r, b, y, NULL) == 0, "stack f64 no dump");
        expect(oracle_stack_window_f32(steps, in0, hidden, layers, x, w, r, b, yf, NULL) == 0, "stack f32");
        double *gates = malloc(sizeof(double) * steps * 2 * g);
        expect(oracle_projection_f64(steps, in0, hidden, x, NULL, w, b, gates) == 0, "projection f64");
        expect(oracle_recurrence_f64(steps, hidden, gates, r, y) == 0, "recurrence f64");
        if (layers > 1) /* layer 1's projection of layer 0's double output */
            expect(oracle_projection_f64(steps, width, hidden, NULL, y, w + (size_t)2 * g * in0, b + 4 * g, gates) == 0,
                   "projection f64 from doubles");
        float *gf = malloc(sizeof(float) * steps * 2 * g);
        expect(oracle_projection_f32(steps, in0, hidden, x, NULL, w, b, gf) == 0, "projection f32");
        expect(oracle_recurrence_f32(steps, hidden, gf, r, yf) == 0, "recurrence f32");
        free(x), free(w), free(r), free(b), free(y), free(dump), free(yf), free(gates), free(gf);
    }
    /* the heads: 5 rows of 12 inputs through 6, 5 and 3 units; and zero rows */
    {
        float *y = rand_array(5 * 12), *w0 = rand_array(12 * 6), *b0 = rand_array(6), *w1 = rand_array(6 * 5);
        float *b1 = rand_array(5), *w2 = rand_array(5 * 3), *b2 = rand_array(3);
        double out[15];
        expect(oracle_heads_f64(5, 12, 6, 5, 3, 0.01, y, NULL, w0, b0, w1, b1, w2, b2, out) == 0, "heads");
        expect(finite_d(out, 15), "heads finite");
        expect(oracle_heads_f64(0, 12, 6, 5, 3, 0.01, y, NULL, w0, b0, w1, b1, w2, b2, out) == 0, "heads 0 rows");
        expect(oracle_heads_f64(5, 12, 6, 5, 3, 0.01, NULL, NULL, w0, b0, w1, b1, w2, b2, out) == -1, "heads NULL");
        free(y), free(w0), free(b0), free(w1), free(b1), free(w2), free(b2);
    }
    /* rejected arguments */
    double d[4];
    float f[4] = {0, 0, 0, 0};
    expect(oracle_stack_window_f64(1, 1, 1, 1, NULL, f, f, f, d, NULL) == -1, "stack NULL x");
    expect(oracle_projection_f64(-1, 1, 1, f, NULL, f, f, d) == -1, "projection negative rows");
    expect(oracle_recurrence_f64(1, 0, d, f, d) == -1, "recurrence zero hidden");
    printf("oracle checks: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
