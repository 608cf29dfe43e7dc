/*
 * fastcall.c -- argument marshalling for the Python binding's hot calls.
 *
 * The two per-step entry points of librmsnorm.so (rmsnorm_fwd and
 * add_rmsnorm_fwd, include/rmsnorm.h) called straight from Python ints and
 * floats through the CPython C API, instead of through ctypes' per-argument
 * conversion.  The module does no arithmetic and no validation of its own:
 * it converts the arguments, calls the library (opened with dlopen at the
 * path the binding gives, which is the instance ctypes already loaded) and
 * returns its status code.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <dlfcn.h>
#include <stdint.h>

typedef int (*rmsnorm_fwd_t)(void*, const void*, const void*, int64_t, int64_t, float, int, void*);
typedef int (*add_rmsnorm_fwd_t)(void*, void*, const void* const*, int, const void*, int64_t,
                                 int64_t, float, int, void*);

static rmsnorm_fwd_t p_rmsnorm_fwd;
static add_rmsnorm_fwd_t p_add_rmsnorm_fwd;

#define KMAX 16

/* open(path): resolve the entry points in the library at `path`. */
static PyObject* fc_open(PyObject* self, PyObject* arg) {
  (void)self;
  const char* path = PyUnicode_AsUTF8(arg);
  if (!path) return NULL;
  void* h = dlopen(path, RTLD_NOW | RTLD_GLOBAL);
  if (!h) {
    PyErr_Format(PyExc_OSError, "dlopen(%s) failed: %s", path, dlerror());
    return NULL;
  }
  p_rmsnorm_fwd = (rmsnorm_fwd_t)dlsym(h, "rmsnorm_fwd");
  p_add_rmsnorm_fwd = (add_rmsnorm_fwd_t)dlsym(h, "add_rmsnorm_fwd");
  if (!p_rmsnorm_fwd || !p_add_rmsnorm_fwd) {
    PyErr_SetString(PyExc_OSError, "librmsnorm.so lacks rmsnorm_fwd / add_rmsnorm_fwd");
    return NULL;
  }
  Py_RETURN_NONE;
}

static int as_ptr(PyObject* o, void** p) {
  *p = o == Py_None ? NULL : PyLong_AsVoidPtr(o);
  return !(*p == NULL && PyErr_Occurred());
}

/* rmsnorm_fwd(out, x, gamma, rows, hidden, eps, dtype, stream) -> status */
static PyObject* fc_rmsnorm_fwd(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  if (n != 8) {
    PyErr_SetString(PyExc_TypeError, "rmsnorm_fwd takes 8 arguments");
    return NULL;
  }
  void *out, *x, *g, *s;
  if (!as_ptr(a[0], &out) || !as_ptr(a[1], &x) || !as_ptr(a[2], &g) || !as_ptr(a[7], &s))
    return NULL;
  const long long rows = PyLong_AsLongLong(a[3]), hidden = PyLong_AsLongLong(a[4]);
  const double eps = PyFloat_AsDouble(a[5]);
  const long dtype = PyLong_AsLong(a[6]);
  if (PyErr_Occurred()) return NULL;
  return PyLong_FromLong(p_rmsnorm_fwd(out, x, g, rows, hidden, (float)eps, (int)dtype, s));
}

/* add_rmsnorm_fwd(out, residual, partials (sequence of ints), gamma, rows,
   hidden, eps, dtype, stream) -> status */
static PyObject* fc_add_rmsnorm_fwd(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  if (n != 9) {
    PyErr_SetString(PyExc_TypeError, "add_rmsnorm_fwd takes 9 arguments");
    return NULL;
  }
  void *out, *r, *g, *s;
  if (!as_ptr(a[0], &out) || !as_ptr(a[1], &r) || !as_ptr(a[3], &g) || !as_ptr(a[8], &s))
    return NULL;
  PyObject* seq = PySequence_Fast(a[2], "partials must be a sequence");
  if (!seq) return NULL;
  const Py_ssize_t k = PySequence_Fast_GET_SIZE(seq);
  /* every k is passed through: the library checks its range */
  const void* stack[KMAX];
  const void** parts = k <= KMAX ? stack : (const void**)PyMem_Malloc(sizeof(void*) * (size_t)k);
  if (!parts) {
    Py_DECREF(seq);
    return PyErr_NoMemory();
  }
  int ok = 1;
  for (Py_ssize_t i = 0; i < k && ok; ++i) {
    void* p;
    ok = as_ptr(PySequence_Fast_GET_ITEM(seq, i), &p);
    parts[i] = p;
  }
  Py_DECREF(seq);
  const long long rows = PyLong_AsLongLong(a[4]), hidden = PyLong_AsLongLong(a[5]);
  const double eps = PyFloat_AsDouble(a[6]);
  const long dtype = PyLong_AsLong(a[7]);
  PyObject* ret = NULL;
  if (ok && !PyErr_Occurred())
    ret = PyLong_FromLong(p_add_rmsnorm_fwd(out, r, parts, (int)k, g, rows, hidden, (float)eps,
                                            (int)dtype, s));
  if (parts != stack) PyMem_Free(parts);
  return ret;
}

static PyMethodDef methods[] = {
    {"open", fc_open, METH_O, "resolve the library's entry points"},
    {"rmsnorm_fwd", (PyCFunction)(void (*)(void))fc_rmsnorm_fwd, METH_FASTCALL, "rmsnorm_fwd"},
    {"add_rmsnorm_fwd", (PyCFunction)(void (*)(void))fc_add_rmsnorm_fwd, METH_FASTCALL,
     "add_rmsnorm_fwd"},
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_fastcall", NULL, -1, methods,
                                    NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__fastcall(void) { return PyModule_Create(&module); }
