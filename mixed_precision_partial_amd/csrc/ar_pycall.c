/*
 * ar_pycall.c -- a CPython type that holds one reduce call of the C ABI with
 * every argument already converted, so that a Python caller can issue the
 * same call again for the cost of one C call.  It does no arithmetic and no
 * validation of its own: each invocation calls ar_reduce / ar_reduce_add of
 * libmpp_ar.so through the function pointer it was given, and the library
 * validates every call.  Built with the host C compiler into
 * _ar_fast<EXT_SUFFIX> beside the binding; the binding falls back to ctypes
 * when it is absent.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stddef.h>
#include <stdint.h>

typedef int (*reduce_fn)(void *ctx, void *const *dst, const void *const *srcs, int R, size_t n, int dst_type,
                         int wire_type, unsigned mode, void *hip_stream);
typedef int (*reduce_add_fn)(void *ctx, void *const *dst, const void *const *srcs, int R, size_t n, int dst_type,
                             int wire_type, unsigned mode, const void *residual, size_t residual_len,
                             void *hip_stream);

typedef struct {
    PyObject_HEAD
    void *fn;              /* ar_reduce or ar_reduce_add */
    int with_residual;
    void *ctx;
    void *const *dst;
    const void *const *srcs;
    int R;
    size_t n;
    int dst_type;
    int wire_type;
    unsigned mode;
    const void *residual;
    size_t residual_len;
    void *stream;
    PyObject *keep;        /* objects that own the pointer arrays */
} BoundCall;

static void bound_dealloc(BoundCall *self) {
    Py_XDECREF(self->keep);
    Py_TYPE(self)->tp_free((PyObject *)self);
}

static PyObject *bound_call(BoundCall *self, PyObject *args, PyObject *kwargs) {
    if (PyTuple_GET_SIZE(args) != 0 || (kwargs != NULL && PyDict_GET_SIZE(kwargs) != 0)) {
        PyErr_SetString(PyExc_TypeError, "a bound call takes no arguments");
        return NULL;
    }
    int rc;
    if (self->with_residual) {
        rc = ((reduce_add_fn)self->fn)(self->ctx, self->dst, self->srcs, self->R, self->n, self->dst_type,
                                       self->wire_type, self->mode, self->residual, self->residual_len,
                                       self->stream);
    } else {
        rc = ((reduce_fn)self->fn)(self->ctx, self->dst, self->srcs, self->R, self->n, self->dst_type,
                                   self->wire_type, self->mode, self->stream);
    }
    return PyLong_FromLong(rc);
}

static PyTypeObject BoundCallType = {
    PyVarObject_HEAD_INIT(NULL, 0)
    .tp_name = "_ar_fast.BoundCall",
    .tp_basicsize = sizeof(BoundCall),
    .tp_dealloc = (destructor)bound_dealloc,
    .tp_call = (ternaryfunc)bound_call,
    .tp_flags = Py_TPFLAGS_DEFAULT,
    .tp_doc = "one reduce call with its arguments converted once; call it to enqueue it again",
};

/* bind(fn, with_residual, ctx, dst, srcs, R, n, dst_type, wire_type, mode, residual,
 *      residual_len, stream, keep) -- addresses as Python ints */
static PyObject *bind(PyObject *module, PyObject *args) {
    (void)module;
    unsigned long long fn, ctx, dst, srcs, residual, stream;
    unsigned long long n, residual_len;
    int with_residual, R, dst_type, wire_type;
    unsigned int mode;
    PyObject *keep;
    if (!PyArg_ParseTuple(args, "KpKKKiKiiIKKKO", &fn, &with_residual, &ctx, &dst, &srcs, &R, &n, &dst_type,
                          &wire_type, &mode, &residual, &residual_len, &stream, &keep)) {
        return NULL;
    }
    if (fn == 0) {
        PyErr_SetString(PyExc_ValueError, "null function pointer");
        return NULL;
    }
    BoundCall *self = PyObject_New(BoundCall, &BoundCallType);
    if (self == NULL) return NULL;
    self->fn = (void *)(uintptr_t)fn;
    self->with_residual = with_residual;
    self->ctx = (void *)(uintptr_t)ctx;
    self->dst = (void *const *)(uintptr_t)dst;
    self->srcs = (const void *const *)(uintptr_t)srcs;
    self->R = R;
    self->n = (size_t)n;
    self->dst_type = dst_type;
    self->wire_type = wire_type;
    self->mode = mode;
    self->residual = (const void *)(uintptr_t)residual;
    self->residual_len = (size_t)residual_len;
    self->stream = (void *)(uintptr_t)stream;
    Py_INCREF(keep);
    self->keep = keep;
    return (PyObject *)self;
}

static PyMethodDef methods[] = {
    {"bind", bind, METH_VARARGS, "bind one call of ar_reduce / ar_reduce_add"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef moduledef = {
    PyModuleDef_HEAD_INIT, "_ar_fast", "pre-converted calls of the reduce library", -1, methods,
    NULL, NULL, NULL, NULL,
};

PyMODINIT_FUNC PyInit__ar_fast(void) {
    if (PyType_Ready(&BoundCallType) < 0) return NULL;
    PyObject *m = PyModule_Create(&moduledef);
    if (m == NULL) return NULL;
    Py_INCREF(&BoundCallType);
    if (PyModule_AddObject(m, "BoundCall", (PyObject *)&BoundCallType) < 0) {
        Py_DECREF(&BoundCallType);
        Py_DECREF(m);
        return NULL;
    }
    return m;
}
